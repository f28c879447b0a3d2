// Top-k token selection over fp32 scores: the k largest of each row, ties to
// the lower token index, written in ascending index order, -1 padded.
//
// ("Attention Optimizations", "Computation Path": indices = topk(I, 2048);
// "Caveats": a top-k over the whole context is expensive, so it is a radix
// select, not a sort.)
//
// Every row is cut into chunks of 2048 tokens, one workgroup of 256 threads
// per chunk (thread t holds tokens chunk*2048 + 256 j + t, j < 8), so a batch
// of long rows spreads over the whole chip.  Scores become order-preserving
// unsigned keys (-0.0 folded onto +0.0) and the k-th largest key T is found
// most significant byte first.  Workgroups meet only at kernel boundaries, five
// launches on the same grid, and never add into shared counters: each chunk
// stores its own 256-bin histogram of the current byte (over the keys that
// match the bytes fixed so far), and every workgroup of the next launch sums
// its row's chunk histograms itself, finds the byte holding the k-th largest
// key and how many keys of that bin are still needed (`need`):
//   launch 0: histograms of byte 3;
//   launch l = 1, 2, 3: fix byte 4 - l, histograms of byte 3 - l; launch 3
//             also counts, per chunk, the keys whose top three bytes are
//             already above T's;
//   launch 4 (write): fix byte 0, hence T and `need`.  The same column sums,
//             taken over the chunks before this one only, give the keys above
//             T and equal to T that precede the chunk; ballots rank the keys
//             inside it, and a taken key goes to
//             (keys above T before it) + min(keys equal to T before it, need),
//             so indices come out ascending and ties go to the lower index.
// Workgroup 0 of a row records each decision for the next launch.  Rows with
// seq_len <= k are written directly by the first launch.  Nothing in the
// workspace has to be cleared beforehand.  The first level's histograms may
// come from the producer of the scores instead (the indexer, when its
// workgroups cover exactly these chunks); launch 0 is then skipped.  When
// every row fits one chunk
// (S_max <= 2048, e.g. a selection over 16-token pages), one workgroup owns a
// row and runs the four levels and the write in a single launch, with the
// histograms in LDS.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kTT = 256;             // threads per workgroup
constexpr int kNW = kTT / 64;        // waves per workgroup
constexpr int kKPT = 8;              // keys per thread
constexpr int kChunk = kTT * kKPT;   // tokens per workgroup
static_assert(kChunk == kTopkChunk, "chunk size shared with the indexer");
constexpr int kBins = 256;           // one byte of the key per launch
constexpr int kColBatch = 32;        // chunk histograms loaded per batch

// One row's workspace, in 32-bit words.
struct RowWs {
  uint32_t* h;     // [4][n_chunks][256]: per-chunk histograms of bytes 3, 2, 1, 0
  uint32_t* above; // [n_chunks]: keys whose top three bytes exceed T's
  uint32_t* st;    // [8]: byte 3, need; top 16 bits, need; top 24 bits, need
};

__host__ __device__ inline size_t topk_row_words(int n_chunks) {
  const size_t w = (size_t)n_chunks * (4 * kBins + 1) + 8;
  return (w + 63) & ~(size_t)63;
}

__device__ __forceinline__ RowWs row_ws(const TopkArgs& a, int b) {
  RowWs r;
  r.h = a.ws + (size_t)b * a.row_words;
  r.above = r.h + (size_t)4 * a.n_chunks * kBins;
  r.st = r.above + a.n_chunks;
  return r;
}

// seq_lens outside [0, S_max] are clamped into it
__device__ __forceinline__ int row_len(const TopkArgs& a, int b) {
  return min(max(a.seq_lens[b], 0), a.S_max);
}

// This workgroup's keys, loaded without waiting for the row length (tokens
// past S_max read the row's last entry; `valid_mask` sorts them out).
__device__ __forceinline__ void load_keys(const TopkArgs& a, int b, int c, uint32_t (&key)[kKPT]) {
  const float* row = a.scores + (size_t)b * a.S_max;
  const int t0 = c * kChunk + (int)threadIdx.x;
  float x[kKPT];
#pragma unroll
  for (int j = 0; j < kKPT; ++j) x[j] = row[min(t0 + j * kTT, a.S_max - 1)];
#pragma unroll
  for (int j = 0; j < kKPT; ++j) key[j] = order_key(x[j]);
}

// bit j: token 256 j + t of chunk c lies inside the row
__device__ __forceinline__ uint32_t valid_mask(int c, int L) {
  const int t0 = c * kChunk + (int)threadIdx.x;
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < kKPT; ++j) v |= (uint32_t)(t0 + j * kTT < L) << j;
  return v;
}

// Thread t: column 255 - t of the row's chunk histograms `h` ([n_chunks][256]),
// summed over the chunks < nc (`tot`) and over the chunks < c (`pre`).
// Loads cover chunks < n_load (>= nc); with n_load = n_chunks they need not
// wait for the row length.
__device__ __forceinline__ void column_sums(const uint32_t* h, int n_load, int nc, int c,
                                            uint32_t& tot, uint32_t& pre) {
  const uint32_t* col = h + (kBins - 1 - threadIdx.x);
  tot = 0;
  pre = 0;
  for (int c0 = 0; c0 < n_load; c0 += kColBatch) {
    uint32_t v[kColBatch];
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) v[u] = col[(size_t)min(c0 + u, n_load - 1) * kBins];
#pragma unroll
    for (int u = 0; u < kColBatch; ++u) {
      tot += c0 + u < nc ? v[u] : 0u;
      pre += c0 + u < c ? v[u] : 0u;
    }
  }
}

// Short grids load every chunk's column at once; long rows load only the
// chunks inside the row, which costs a wait for the row length first.
constexpr int kEagerChunks = 64;
__device__ __forceinline__ void row_column_sums(const TopkArgs& a, const uint32_t* h, int L, int c,
                                                uint32_t& tot, uint32_t& pre) {
  const int nc = (L + kChunk - 1) / kChunk;
  if (a.n_chunks <= kEagerChunks)
    column_sums(h, a.n_chunks, nc, c, tot, pre);
  else
    column_sums(h, nc, nc, c, tot, pre);
}

__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) s += red[w];
  __syncthreads();
  return s;
}

// Thread t holds the count of bin 255 - t.  Returns the bin holding the
// need-th largest key counting from the top, and in `rest` how many keys of
// that bin are still needed.  All threads get the same answer.
__device__ __forceinline__ uint32_t find_byte(uint32_t cnt, uint32_t need, uint32_t* wave_tot,
                                              uint32_t* res, uint32_t& rest) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t before = inc - cnt;
#pragma unroll
  for (int w = 0; w < kNW; ++w) before += w < wave ? wave_tot[w] : 0u;
  if (before < need && before + cnt >= need) {
    res[0] = kBins - 1 - threadIdx.x;
    res[1] = need - before;
  }
  __syncthreads();
  rest = res[1];
  return res[0];
}

// Launch LEVEL (0..3): histograms of key byte 3 - LEVEL over the keys that
// match the LEVEL bytes fixed so far.
template <int LEVEL>
__global__ __launch_bounds__(kTT) void topk_digit_kernel(const TopkArgs a) {
  constexpr int kShift = 24 - 8 * LEVEL;
  __shared__ uint32_t hist[kBins], wave_tot[kNW], res[2], red[kNW];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const RowWs w = row_ws(a, b);
  uint32_t key[kKPT];
  load_keys(a, b, c, key);
  uint32_t tot = 0, pre = 0, prev_prefix = 0, prev_need = (uint32_t)a.k;
  const int L = row_len(a, b), K = a.k;
  if (LEVEL > 0) {
    if (LEVEL > 1) {
      prev_prefix = w.st[2 * (LEVEL - 2)];
      prev_need = w.st[2 * (LEVEL - 2) + 1];
    }
    row_column_sums(a, w.h + (size_t)(LEVEL - 1) * a.n_chunks * kBins, L, 0, tot, pre);
  }
  if ((LEVEL == 0 || (LEVEL == 1 && a.hist0_done)) && L <= K) {  // the first launch writes short rows
    int32_t* out = a.idx + (size_t)b * K;
    for (int j = c * kTT + tid; j < K; j += a.n_chunks * kTT) out[j] = j < L ? j : -1;
    return;
  }
  if (L <= K || c * kChunk >= L) return;
  const uint32_t valid = valid_mask(c, L);
  uint32_t prefix = 0;
  if (LEVEL > 0) {
    uint32_t need;
    prefix = (prev_prefix << 8) | find_byte(tot, prev_need, wave_tot, res, need);
    if (c == 0 && tid == 0) {
      w.st[2 * (LEVEL - 1)] = prefix;
      w.st[2 * (LEVEL - 1) + 1] = need;
    }
  }
  hist[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kKPT; ++j) {
    const bool m = ((valid >> j) & 1u) && (LEVEL == 0 || (key[j] >> (kShift + 8)) == prefix);
    hist_add(hist, m, (key[j] >> kShift) & (kBins - 1));
  }
  __syncthreads();
  w.h[((size_t)LEVEL * a.n_chunks + c) * kBins + tid] = hist[tid];
  if (LEVEL == 3) {
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < kKPT; ++j) n += ((valid >> j) & 1u) && (key[j] >> 8) > prefix;
    n = block_sum(n, red);
    if (tid == 0) w.above[c] = n;
  }
}

// Writes the taken keys of chunk c: those above T, and the first `need`
// equal to T in row order, at ranks counted from base_gt / base_eq (the keys
// above / equal to T in the chunks before this one), so that indices come out
// ascending.
__device__ __forceinline__ void rank_and_write(const TopkArgs& a, int b, int c, const uint32_t (&key)[kKPT],
                                               uint32_t valid, uint32_t T, uint32_t need, uint32_t base_gt,
                                               uint32_t base_eq, uint32_t* off_gt, uint32_t* off_eq) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k;
  // per (column j, wave) counts, then exclusive offsets in token order
  uint64_t mg[kKPT], me[kKPT];
#pragma unroll
  for (int j = 0; j < kKPT; ++j) {
    const bool v = (valid >> j) & 1u;
    mg[j] = __ballot(v && key[j] > T);
    me[j] = __ballot(v && key[j] == T);
    if (lane == 0) {
      off_gt[j * kNW + wave] = (uint32_t)__popcll(mg[j]);
      off_eq[j * kNW + wave] = (uint32_t)__popcll(me[j]);
    }
  }
  __syncthreads();
  if (tid < 64) {
    constexpr int kE = kKPT * kNW;  // 32 entries, one per lane
    const uint32_t g = lane < kE ? off_gt[lane] : 0u, e = lane < kE ? off_eq[lane] : 0u;
    uint32_t ig = g, ie = e;
#pragma unroll
    for (int d = 1; d < kE; d <<= 1) {
      const uint32_t yg = __shfl_up(ig, d), ye = __shfl_up(ie, d);
      if (lane >= d) {
        ig += yg;
        ie += ye;
      }
    }
    if (lane < kE) {
      off_gt[lane] = ig - g;
      off_eq[lane] = ie - e;
    }
  }
  __syncthreads();
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int32_t* out = a.idx + (size_t)b * K;
  const int t0 = c * kChunk + tid;
#pragma unroll
  for (int j = 0; j < kKPT; ++j) {
    const bool v = (valid >> j) & 1u;
    const bool gt = v && key[j] > T, eq = v && key[j] == T;
    const uint32_t r_gt = base_gt + off_gt[j * kNW + wave] + (uint32_t)__popcll(mg[j] & below);
    const uint32_t r_eq = base_eq + off_eq[j * kNW + wave] + (uint32_t)__popcll(me[j] & below);
    if (gt || (eq && r_eq < need)) {
      const uint32_t pos = r_gt + min(r_eq, need);
      if (pos < (uint32_t)K) out[pos] = t0 + j * kTT;  // always true when the select is right
    }
  }
}

__global__ __launch_bounds__(kTT) void topk_write_kernel(const TopkArgs a) {
  __shared__ uint32_t wave_tot[kNW], res[2], red[kNW], eq_pre;
  __shared__ uint32_t off_gt[kKPT * kNW], off_eq[kKPT * kNW];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const RowWs w = row_ws(a, b);
  uint32_t key[kKPT];
  load_keys(a, b, c, key);
  const uint32_t p24 = w.st[4], need2 = w.st[5];
  uint32_t ab = 0;  // keys above T's top three bytes in the chunks before this one
  for (int cc = tid; cc < c; cc += kTT) ab += w.above[cc];
  const int L = row_len(a, b), K = a.k;
  uint32_t tot, pre;
  row_column_sums(a, w.h + (size_t)3 * a.n_chunks * kBins, L, c, tot, pre);
  if (L <= K || c * kChunk >= L) return;
  const uint32_t valid = valid_mask(c, L);
  uint32_t need;
  const uint32_t d0 = find_byte(tot, need2, wave_tot, res, need);
  const uint32_t T = (p24 << 8) | d0;
  const uint32_t bin = kBins - 1 - tid;
  if (bin == d0) eq_pre = pre;
  const uint32_t base_gt = block_sum(ab + (bin > d0 ? pre : 0u), red);  // syncs: eq_pre visible
  const uint32_t base_eq = eq_pre;

  rank_and_write(a, b, c, key, valid, T, need, base_gt, base_eq, off_gt, off_eq);
}

// One workgroup per row when the row fits one chunk (S_max <= 2048): the four
// byte levels run in LDS back to back, then the same ranked write, in one
// launch.
__global__ __launch_bounds__(kTT) void topk_single_kernel(const TopkArgs a) {
  __shared__ uint32_t hist[kBins], wave_tot[kNW], res[2];
  __shared__ uint32_t off_gt[kKPT * kNW], off_eq[kKPT * kNW];
  const int b = blockIdx.y, tid = threadIdx.x;
  uint32_t key[kKPT];
  load_keys(a, b, 0, key);
  const int L = row_len(a, b), K = a.k;
  if (L <= K) {
    int32_t* out = a.idx + (size_t)b * K;
    for (int j = tid; j < K; j += kTT) out[j] = j < L ? j : -1;
    return;
  }
  const uint32_t valid = valid_mask(0, L);
  uint32_t prefix = 0, need = (uint32_t)K;
#pragma unroll
  for (int level = 0; level < 4; ++level) {
    const int shift = 24 - 8 * level;
    hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kKPT; ++j) {
      const bool m = ((valid >> j) & 1u) && (level == 0 || (key[j] >> (shift + 8)) == prefix);
      hist_add(hist, m, (key[j] >> shift) & (kBins - 1));
    }
    __syncthreads();
    uint32_t rest;
    prefix = (prefix << 8) | find_byte(hist[kBins - 1 - tid], need, wave_tot, res, rest);
    need = rest;
  }
  rank_and_write(a, b, 0, key, valid, prefix, need, 0u, 0u, off_gt, off_eq);
}

}  // namespace

int64_t topk_row_words_of(int S_max) {
  return (int64_t)topk_row_words((S_max + kChunk - 1) / kChunk);
}

size_t topk_workspace_bytes(int B, int S_max) {
  const int nc = (S_max + kChunk - 1) / kChunk;
  return ((size_t)B * topk_row_words(nc) * 4 + 255) & ~(size_t)255;
}

hipError_t launch_topk(const TopkArgs& a0, hipStream_t s) {
  TopkArgs a = a0;
  a.n_chunks = (a.S_max + kChunk - 1) / kChunk;
  a.row_words = (int64_t)topk_row_words(a.n_chunks);
  const dim3 grid(a.n_chunks, a.B);
  if (a.n_chunks == 1) {
    launch_kernel(topk_single_kernel, grid, kTT, s, a);
    return hipGetLastError();
  }
  if (!a.hist0_done) launch_kernel(topk_digit_kernel<0>, grid, kTT, s, a);
  launch_kernel(topk_digit_kernel<1>, grid, kTT, s, a);
  launch_kernel(topk_digit_kernel<2>, grid, kTT, s, a);
  launch_kernel(topk_digit_kernel<3>, grid, kTT, s, a);
  launch_kernel(topk_write_kernel, grid, kTT, s, a);
  return hipGetLastError();
}

}  // namespace dattn
