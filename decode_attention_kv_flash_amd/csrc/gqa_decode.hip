// Split-K decode attention over a paged KV cache: grouped-query heads,
// optional sliding window plus attention sinks.
//
// One workgroup owns (sequence b, KV head, token split).  The G query heads
// that share the KV head ("All the attentions", section 2) are processed
// together, so every K/V byte is read from HBM exactly once per call.  The
// token set of the query is the window's last `window` tokens plus the first
// `n_sink` sinks ("All the attentions", section 4; "Attention Optimizations",
// "Attention sinks"); tokens outside it are never loaded -- the kernel walks
// a flattened index over the set, not a mask over the cache.
//
// Inside a workgroup each wave streams its own 16-token steps:
//   * a token row of D values is split over LPT lanes in 16-byte pieces, so
//     one wave load instruction reads 64 x 16 B = 1 KiB of consecutive rows
//     of a page (4 KiB per bf16 page per head);
//   * scores are lane-partial dot products (v_dot2_f32_bf16 for bf16: the
//     bf16 products are exact in fp32) summed over the LPT lanes with DPP;
//   * the softmax is the online one ("All the attentions", section 1: a
//     running maximum and running sum, earlier partials rescaled), kept per
//     token row of the wave and merged at the end;
//   * P.V accumulates in fp32 registers.
// A split's result is (o / l, log2-sum-exp); lse_combine merges splits.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 16;  // tokens per wave step

template <bool BF16, int D>
struct GqaShape {
  static constexpr int ESZ = BF16 ? 2 : 4;   // bytes per element
  static constexpr int VEC = 16 / ESZ;       // elements per 16-byte piece
  static constexpr int LPT = D / VEC;        // lanes per token row
  static constexpr int TPL = 64 / LPT;       // token rows per wave load
  static constexpr int NI = kStep / TPL;     // loads per step
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "row split");
};

template <bool BF16, int VEC>
__device__ __forceinline__ void widen(const uint4& x, float (&f)[VEC]) {
  if constexpr (BF16) {
    f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
    f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
    f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z);
    f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
  } else {
    f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
  }
}

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kThreads) void gqa_split_kernel(const GqaArgs a) {
  using S = GqaShape<BF16, D>;
  constexpr int VEC = S::VEC, LPT = S::LPT, TPL = S::TPL, NI = S::NI;
  const float NEG_INF = -__builtin_inff();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;

  // Token set of this sequence, flattened: f in [0, N) maps to position
  // t = f for the sinks kept outside the window, else into the window.
  const int L = a.seq_lens[b];
  int s_cnt = 0, w_start = 0, N = L;
  if (a.window > 0 && a.window < L) {
    w_start = L - a.window;
    s_cnt = min(a.n_sink, w_start);
    N = s_cnt + a.window;
  }
  const int per = ((N + a.num_splits - 1) / a.num_splits + kStep - 1) / kStep * kStep;
  const int f_begin = split * per;
  const int f_end = min(N, f_begin + per);
  const int n_steps = f_end > f_begin ? (f_end - f_begin + kStep - 1) / kStep : 0;

  // This lane's 16-byte piece of the G query rows.
  uint4 qv[G];
  {
    const char* qb = (const char*)a.q + ((size_t)(b * a.Hq + kvh * G) * D + c * VEC) * S::ESZ;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *(const uint4*)(qb + (size_t)h * D * S::ESZ);
  }

  float m[G], l[G], o[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = NEG_INF;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
  }

  const size_t head_stride = (size_t)a.page_size * D;
  const size_t page_stride = (size_t)a.Hkv * head_stride;
  const char* kb = (const char*)a.k;
  const char* vb = (const char*)a.v;
  const int32_t* pt = a.page_table ? a.page_table + (size_t)b * a.max_pages : nullptr;
  const size_t contig_base = ((size_t)b * a.Hkv + kvh) * head_stride;

  for (int step = wave; step < n_steps; step += kWaves) {
    uint4 kr[NI], vr[NI];
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int f = f_begin + step * kStep + i * TPL + r;
      valid[i] = f < f_end;
      const int t = f < s_cnt ? f : w_start + (f - s_cnt);
      size_t off;
      if (pt) {
        const int phys = valid[i] ? pt[t >> a.log2_page] : 0;
        off = (size_t)phys * page_stride + (size_t)kvh * head_stride +
              (size_t)(t & (a.page_size - 1)) * D;
      } else {
        off = contig_base + (size_t)t * D;
      }
      off = (off + (size_t)c * VEC) * S::ESZ;
      if (valid[i]) {
        kr[i] = *(const uint4*)(kb + off);
        vr[i] = *(const uint4*)(vb + off);
      } else {
        kr[i] = make_uint4(0u, 0u, 0u, 0u);
        vr[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // scores s[i][h], log2 units
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
        if constexpr (BF16) {
          acc = dot2_bf16(kr[i].x, qv[h].x, acc);
          acc = dot2_bf16(kr[i].y, qv[h].y, acc);
          acc = dot2_bf16(kr[i].z, qv[h].z, acc);
          acc = dot2_bf16(kr[i].w, qv[h].w, acc);
        } else {
          acc = __uint_as_float(kr[i].x) * __uint_as_float(qv[h].x);
          acc = fmaf(__uint_as_float(kr[i].y), __uint_as_float(qv[h].y), acc);
          acc = fmaf(__uint_as_float(kr[i].z), __uint_as_float(qv[h].z), acc);
          acc = fmaf(__uint_as_float(kr[i].w), __uint_as_float(qv[h].w), acc);
        }
        acc = group_sum<LPT>(acc) * a.scale_log2;
        s[i][h] = valid[i] ? acc : NEG_INF;
      }
    }

    // online softmax update per token row
    float p[NI][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx = fmaxf(mx, s[i][h]);
      const float mn = fmaxf(m[h], mx);
      const float mu = mn == NEG_INF ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - mu);
      m[h] = mn;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        p[i][h] = fast_exp2(s[i][h] - mu);
        ps += p[i][h];
      }
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] *= alpha;
    }

    // P.V
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[VEC];
      widen<BF16, VEC>(vr[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(p[i][h], vf[e], o[h][e]);
      }
    }
  }

  // merge the TPL token rows of the wave (lanes c, c+LPT, ...)
#pragma unroll
  for (int d = LPT; d < 64; d <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], d);
      const float lo = __shfl_xor(l[h], d);
      const float mn = fmaxf(m[h], mo);
      const float mu = mn == NEG_INF ? 0.f : mn;
      const float a1 = fast_exp2(m[h] - mu), a2 = fast_exp2(mo - mu);
      l[h] = l[h] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] = o[h][e] * a1 + __shfl_xor(o[h][e], d) * a2;
      m[h] = mn;
    }
  }

  // merge the waves
  __shared__ float sm_m[kWaves][G], sm_l[kWaves][G];
  __shared__ float sm_o[kWaves][G][D];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_o[wave][h][c * VEC + e] = o[h][e];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    const float mu = M == NEG_INF ? 0.f : M;
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm_m[w][h] - mu);
      lsum += sm_l[w][h] * f;
      acc += sm_o[w][h][d] * f;
    }
    const float val = lsum > 0.f ? acc / lsum : 0.f;
    const float lse2 = lsum > 0.f ? M + __log2f(lsum) : NEG_INF;
    const size_t row = (size_t)b * a.Hq + (size_t)kvh * G + h;
    if (a.num_splits == 1) {
      if constexpr (BF16) ((uint16_t*)a.out)[row * D + d] = f32_to_bf16(val);
      else ((float*)a.out)[row * D + d] = val;
      if (d == 0 && a.lse) a.lse[row] = lse2 == NEG_INF ? NEG_INF : lse2 * kLn2;
    } else {
      a.part_o[(row * a.num_splits + split) * D + d] = val;
      if (d == 0) a.part_lse[row * a.num_splits + split] = lse2;
    }
  }
}

template <bool BF16, int D>
hipError_t launch_d(const GqaArgs& a, hipStream_t s) {
  dim3 grid(a.num_splits, a.Hkv, a.B), block(kThreads);
  switch (a.G) {
    case 1: gqa_split_kernel<BF16, D, 1><<<grid, block, 0, s>>>(a); break;
    case 2: gqa_split_kernel<BF16, D, 2><<<grid, block, 0, s>>>(a); break;
    case 4: gqa_split_kernel<BF16, D, 4><<<grid, block, 0, s>>>(a); break;
    case 8: gqa_split_kernel<BF16, D, 8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Merge split partials (o_j normalised, lse_j in log2 units):
// lse = max + log2 sum_j 2^(lse_j - max); o = sum_j 2^(lse_j - lse) o_j.
template <bool BF16>
__global__ __launch_bounds__(256) void lse_combine_kernel(const CombineArgs a) {
  const float NEG_INF = -__builtin_inff();
  const int row = blockIdx.x;
  const float* pl = a.part_lse + (size_t)row * a.splits;
  float M = NEG_INF;
  for (int j = 0; j < a.splits; ++j) M = fmaxf(M, pl[j]);
  const float mu = M == NEG_INF ? 0.f : M;
  float wsum = 0.f;
  for (int j = 0; j < a.splits; ++j) wsum += fast_exp2(pl[j] - mu);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const float* po = a.part_o + (size_t)row * a.splits * a.D;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < a.splits; ++j) acc = fmaf(fast_exp2(pl[j] - mu), po[(size_t)j * a.D + d], acc);
    const float val = acc * inv;
    if constexpr (BF16) ((uint16_t*)a.out)[(size_t)row * a.D + d] = f32_to_bf16(val);
    else ((float*)a.out)[(size_t)row * a.D + d] = val;
  }
  if (threadIdx.x == 0 && a.lse) a.lse[row] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : NEG_INF;
}

}  // namespace

hipError_t launch_gqa(const GqaArgs& a, hipStream_t s) {
  if (a.bf16) {
    if (a.D == 64) return launch_d<true, 64>(a, s);
    if (a.D == 128) return launch_d<true, 128>(a, s);
  } else {
    if (a.D == 64) return launch_d<false, 64>(a, s);
    if (a.D == 128) return launch_d<false, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int threads = a.D >= 256 ? 256 : a.D;
  if (a.bf16) lse_combine_kernel<true><<<a.rows, threads, 0, s>>>(a);
  else lse_combine_kernel<false><<<a.rows, threads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dattn
