/*
 * Plain CPU oracle for single-token decode attention over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * kernels.
 *
 * Every routine here is the definition of the result written out, in double
 * precision (or exact 64-bit integers for the indexer), with no blocking,
 * fusion or reordering:
 *
 *   attention (GQA / sliding window + sinks / MLA / sparse MLA):
 *     two passes per output row -- first every score and their maximum, then
 *     the exponentials, their sum and the weighted sum of values -- which is
 *     the standard softmax attention the eager reference code computes
 *     ("Overview of Attention Mechanism", GQA "Code": matmul with the scaled
 *     keys, softmax, matmul with the values).  FlashAttention-style kernels
 *     reach the same result by an online softmax ("All the attentions",
 *     section 1).
 *   indexer:  I_t = sum_h w_h * ReLU(q_h . k_t), all in int64
 *     ("Attention Optimizations", "DSA: DeepSeek Sparse Attention",
 *     "Computation Path": per-head indexer dot products mixed by per-head
 *     weights; the ReLU and the sum over heads are this library's reading of
 *     the per-head mixing weight).
 *   top-k:    a full sort of (score descending, index ascending); the first
 *     min(k, L) entries are returned in ascending index order, padded with -1.
 *
 * Parallelism: OpenMP over independent output rows only.
 *
 * Element types: 0 = fp32, 1 = bf16 given as raw 16-bit patterns, 2 = fp8
 * e4m3 (the OCP "e4m3fn" format: 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits, subnormals at exponent 0, no infinities, S.1111.111 = NaN)
 * given as raw bytes.  A bf16 value widens exactly to fp32 by a 16-bit left
 * shift, an e4m3 value is decoded exactly from its fields, and fp32 widens
 * exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8_E4M3 2

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOTINT (-2)
#define ORC_ENOMEM (-3)

/* e4m3 byte -> value: (-1)^s 2^(e-7) (1 + m/8), or 2^-6 (m/8) when e = 0. */
static double e4m3_value(uint8_t x) {
  const int sign = x >> 7, e = (x >> 3) & 15, m = x & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return sign ? -v : v;
}

double oracle_e4m3_value(int x) { return e4m3_value((uint8_t)x); }

static double elem(const void* p, int dtype, int64_t i) {
  if (dtype == ORC_F32) return (double)((const float*)p)[i];
  if (dtype == ORC_FP8_E4M3) return e4m3_value(((const uint8_t*)p)[i]);
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int oracle_version(void) { return 1; }

/*
 * Token set of a decode query at position L-1 over L cached tokens.
 *
 * window <= 0: every cached token.  Otherwise the last `window` tokens
 * (positions t with t > (L-1) - window, the sliding-window mask of
 * "All the attentions", section 4) together with the first `n_sink` tokens
 * (StreamingLLM's attention sinks, "Attention Optimizations", "Attention
 * sinks").  The two parts are a union: no token is counted twice.
 */
static int attends(int t, int L, int window, int n_sink) {
  if (window <= 0) return 1;
  if (t > (L - 1) - window) return 1;
  return t < n_sink;
}

/*
 * Grouped-query decode attention.
 *   q       [B, Hq, D]
 *   k, v    [B, Hkv, S_max, D] in logical token order (no paging here)
 *   query head h reads KV head h / (Hq / Hkv): consecutive query heads share,
 *   as repeat_interleave / repeat_kv lay them out ("All the attentions",
 *   section 2; "Overview of Attention Mechanism", GQA "Code").
 *   sink    NULL, or one logit per query head [Hq] (natural-log units): an
 *           extra term exp(sink[h]) in the softmax denominator whose value is
 *           zero -- the explicit learned sink logit ("Attention
 *           Optimizations", "Attention sinks"); sink = 0 is the zero sink of
 *           softmax-off-by-one, a token whose key and value are zero vectors
 *           ("Overview of Attention Mechanism", StreamingLLM / attention
 *           sink).  Then o = sum_t e^{s_t} v_t / (e^{sink} + sum_t e^{s_t}).
 * rows: flat row ids b*Hq + h to compute (NULL = all B*Hq, in order).
 * out [n_rows, D], lse [n_rows] (natural log of the softmax denominator, the
 * sink term included; -inf and zeros for an empty set without a sink).
 */
static int gqa_impl(const void* q, const void* k, const void* v, int dtype,
                    int B, int Hq, int Hkv, int D, int S_max,
                    const int32_t* seq_lens, int window, int n_sink, const double* sink,
                    double scale, const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return ORC_EINVAL;
  if (!rows) n_rows = (int64_t)B * Hq;
  const int G = Hq / Hkv;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int b = (int)(row / Hq), h = (int)(row % Hq), kvh = h / G;
    const int L = seq_lens[b];
    double* o = out + r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (L < 0 || L > S_max || b >= B) {
#pragma omp atomic write
      err = ORC_EINVAL;
      continue;
    }
    double* s = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
    if (!s) {
#pragma omp atomic write
      err = ORC_ENOMEM;
      continue;
    }
    const int64_t qbase = ((int64_t)b * Hq + h) * D;
    const int64_t kvbase = ((int64_t)b * Hkv + kvh) * (int64_t)S_max * D;
    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
      if (!attends(t, L, window, n_sink)) continue;
      double acc = 0.0;
      for (int d = 0; d < D; ++d)
        acc += elem(q, dtype, qbase + d) * elem(k, dtype, kvbase + (int64_t)t * D + d);
      s[t] = scale * acc;
      if (s[t] > m) m = s[t];
    }
    if (sink && sink[h] > m) m = sink[h];
    /* pass 2: exponentials, their sum, weighted values */
    double l = sink ? exp(sink[h] - m) : 0.0;
    for (int t = 0; t < L; ++t) {
      if (!attends(t, L, window, n_sink)) continue;
      const double p = exp(s[t] - m);
      l += p;
      for (int d = 0; d < D; ++d) o[d] += p * elem(v, dtype, kvbase + (int64_t)t * D + d);
    }
    if (l > 0.0) {
      for (int d = 0; d < D; ++d) o[d] /= l;
      lse[r] = m + log(l);
    } else {
      lse[r] = -INFINITY;
    }
    free(s);
  }
  return err;
}

int oracle_gqa(const void* q, const void* k, const void* v, int dtype,
               int B, int Hq, int Hkv, int D, int S_max,
               const int32_t* seq_lens, int window, int n_sink, double scale,
               const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  return gqa_impl(q, k, v, dtype, B, Hq, Hkv, D, S_max, seq_lens, window, n_sink, NULL, scale,
                  rows, n_rows, out, lse);
}

int oracle_gqa_sink(const void* q, const void* k, const void* v, int dtype,
                    int B, int Hq, int Hkv, int D, int S_max,
                    const int32_t* seq_lens, int window, int n_sink, const double* sink,
                    double scale, const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (!sink) return ORC_EINVAL;
  return gqa_impl(q, k, v, dtype, B, Hq, Hkv, D, S_max, seq_lens, window, n_sink, sink, scale,
                  rows, n_rows, out, lse);
}

/*
 * Absorbed MLA decode attention over the latent cache.
 *   q       [B, H, Dc + Dr]   absorbed query: [W_UK^T q_nope ; q_pe]
 *   latent  [B, S_max, Dc + Dr], each row [c_KV (Dc) ; k_pe (Dr)]
 *   score   s_t = scale * q . latent_t over all Dc + Dr entries
 *   output  o = sum_t p_t latent_t[0:Dc] / sum_t p_t        (out [n_rows, Dc])
 * ("Attention Optimizations", "DSA: DeepSeek Sparse Attention" and
 * "Computation Path": the cached row is cat(c_KV, k_pe) of 512 + 64 values;
 * "Overview of Attention Mechanism", MLA "Method": W_UK folds into the query
 * and W_UV into the output projection, so no per-head key or value is built.)
 *
 * Token set: with idx == NULL, tokens [0, seq_lens[b]).  With idx != NULL
 * (sparse MLA), exactly the entries idx[b*k_sel + j] >= 0, j < k_sel, in the
 * given order (an entry listed twice counts twice); seq_lens is then unused.
 */
int oracle_mla(const void* q, const void* latent, int dtype, int B, int H, int Dc, int Dr,
               int S_max, const int32_t* seq_lens, const int32_t* idx, int k_sel,
               double scale, const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (B <= 0 || H <= 0 || Dc <= 0 || Dr < 0) return ORC_EINVAL;
  if (!idx && !seq_lens) return ORC_EINVAL;
  if (!rows) n_rows = (int64_t)B * H;
  const int Dq = Dc + Dr;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t row = rows ? rows[r] : r;
    const int b = (int)(row / H), h = (int)(row % H);
    double* o = out + r * Dc;
    for (int d = 0; d < Dc; ++d) o[d] = 0.0;
    const int n = idx ? k_sel : seq_lens[b];
    if (n < 0 || (!idx && n > S_max)) {
#pragma omp atomic write
      err = ORC_EINVAL;
      continue;
    }
    double* s = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
    if (!s) {
#pragma omp atomic write
      err = ORC_ENOMEM;
      continue;
    }
    const int64_t qbase = ((int64_t)b * H + h) * Dq;
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      const int t = idx ? idx[(int64_t)b * k_sel + j] : j;
      if (t < 0) continue;
      if (t >= S_max) {
#pragma omp atomic write
        err = ORC_EINVAL;
        continue;
      }
      const int64_t cbase = ((int64_t)b * S_max + t) * Dq;
      double acc = 0.0;
      for (int d = 0; d < Dq; ++d) acc += elem(q, dtype, qbase + d) * elem(latent, dtype, cbase + d);
      s[j] = scale * acc;
      if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < n; ++j) {
      const int t = idx ? idx[(int64_t)b * k_sel + j] : j;
      if (t < 0 || t >= S_max) continue;
      const int64_t cbase = ((int64_t)b * S_max + t) * Dq;
      const double p = exp(s[j] - m);
      l += p;
      for (int d = 0; d < Dc; ++d) o[d] += p * elem(latent, dtype, cbase + d);
    }
    if (l > 0.0) {
      for (int d = 0; d < Dc; ++d) o[d] /= l;
      lse[r] = m + log(l);
    } else {
      lse[r] = -INFINITY;
    }
    free(s);
  }
  return err;
}

static int is_integer(double x) { return isfinite(x) && floor(x) == x; }

/*
 * Lightning-indexer scores in exact integer arithmetic.
 *   q_i [B, Hi, Di], k_i [B, S_max, Di] (dtype), w [B, Hi] fp32
 *   scores[b, t] = sum_h w[b,h] * max(0, sum_d q_i[b,h,d] * k_i[b,t,d])
 *   for t < seq_lens[b]; INT64_MIN for t >= seq_lens[b].
 * Every input must be integer-valued (returns ORC_ENOTINT otherwise), so the
 * result is exact and independent of summation order.
 */
int oracle_indexer(const void* q_i, const float* w, const void* k_i, int dtype,
                   int B, int Hi, int Di, int S_max, const int32_t* seq_lens, int64_t* scores) {
  if (B <= 0 || Hi <= 0 || Di <= 0 || S_max <= 0) return ORC_EINVAL;
  int err = ORC_OK;
  for (int64_t i = 0; i < (int64_t)B * Hi * Di; ++i)
    if (!is_integer(elem(q_i, dtype, i))) return ORC_ENOTINT;
  for (int64_t i = 0; i < (int64_t)B * Hi; ++i)
    if (!is_integer((double)w[i])) return ORC_ENOTINT;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] < 0 || seq_lens[b] > S_max) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t bt = 0; bt < (int64_t)B * S_max; ++bt) {
    const int b = (int)(bt / S_max), t = (int)(bt % S_max);
    if (t >= seq_lens[b]) {
      scores[bt] = INT64_MIN;
      continue;
    }
    int64_t kv[4096];
    int ok = Di <= 4096;
    for (int d = 0; ok && d < Di; ++d) {
      const double x = elem(k_i, dtype, ((int64_t)b * S_max + t) * Di + d);
      if (!is_integer(x)) ok = 0;
      else kv[d] = (int64_t)x;
    }
    if (!ok) {
#pragma omp atomic write
      err = ORC_ENOTINT;
      scores[bt] = INT64_MIN;
      continue;
    }
    int64_t total = 0;
    for (int h = 0; h < Hi; ++h) {
      int64_t dot = 0;
      for (int d = 0; d < Di; ++d)
        dot += (int64_t)elem(q_i, dtype, ((int64_t)b * Hi + h) * Di + d) * kv[d];
      if (dot > 0) total += (int64_t)w[(int64_t)b * Hi + h] * dot;
    }
    scores[bt] = total;
  }
  return err;
}

typedef struct {
  double score;
  int32_t index;
} keyed;

/* larger score first; equal scores: lower index first */
static int cmp_keyed(const void* a, const void* b) {
  const keyed* x = (const keyed*)a;
  const keyed* y = (const keyed*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->index > y->index) - (x->index < y->index);
}

static int cmp_i32(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Top-k token selection: the k largest scores among t < seq_lens[b], ties to
 * the lower index; written ascending, -1 padded when k > seq_lens[b].
 * ("Attention Optimizations", "Computation Path": the indexer keeps the
 * top 2048 scores; "Long context, KV eviction and sparse attention", "Sparse
 * attention": exact per-query top-k selection.)
 * kind 0: scores are int64; kind 1: scores are fp32 (NaN rejected; -0.0 and
 * +0.0 compare equal, as numbers).
 */
int oracle_topk(const void* scores, int kind, int B, int S_max, const int32_t* seq_lens, int k,
                int32_t* idx) {
  if (B <= 0 || S_max <= 0 || k <= 0) return ORC_EINVAL;
  int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    const int L = seq_lens[b];
    int32_t* o = idx + (int64_t)b * k;
    for (int j = 0; j < k; ++j) o[j] = -1;
    if (L < 0 || L > S_max) {
#pragma omp atomic write
      err = ORC_EINVAL;
      continue;
    }
    if (L == 0) continue;
    keyed* a = (keyed*)malloc(sizeof(keyed) * L);
    if (!a) {
#pragma omp atomic write
      err = ORC_ENOMEM;
      continue;
    }
    int bad = 0;
    for (int t = 0; t < L; ++t) {
      const int64_t i = (int64_t)b * S_max + t;
      a[t].score = kind == 0 ? (double)((const int64_t*)scores)[i] : (double)((const float*)scores)[i];
      a[t].index = t;
      if (isnan(a[t].score)) bad = 1;
    }
    if (bad) {
#pragma omp atomic write
      err = ORC_EINVAL;
      free(a);
      continue;
    }
    qsort(a, (size_t)L, sizeof(keyed), cmp_keyed);
    const int n = k < L ? k : L;
    for (int j = 0; j < n; ++j) o[j] = a[j].index;
    qsort(o, (size_t)n, sizeof(int32_t), cmp_i32);
    free(a);
  }
  return err;
}
