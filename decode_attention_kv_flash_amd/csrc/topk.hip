// Top-k token selection over fp32 scores: the k largest of each row, ties to
// the lower token index, written in ascending index order, -1 padded.
//
// ("Attention Optimizations", "Computation Path": indices = topk(I, 2048);
// "Caveats": a top-k over the whole context is expensive, so it is a radix
// select, not a sort.)  One workgroup of 1024 threads per row, which reads
// the row once and keeps it on chip -- 32 columns of 1024 keys in registers,
// up to 32 more in LDS -- so every later pass runs from registers and LDS:
//   1. scores become order-preserving unsigned keys (-0.0 folded onto +0.0);
//      column c, thread t holds token 1024 c + t;
//   2. the keys' min and max fix the range; the select then resolves the
//      offset v = key - min most significant digit first, 12 bits a pass: a
//      4096-bin histogram in LDS of the keys that match the digits fixed so
//      far (a wave whose keys share one bin adds its count with one atomic),
//      a block scan from the top finds the digit holding the k-th largest and
//      how many keys equal to the threshold T are still needed (`need`);
//      integer-valued scores resolve in one or two passes;
//   3. an ordered compaction: per column of 1024 tokens, ballots count the
//      keys above T and the keys equal to T per wave; column and wave offsets
//      in LDS give each key its rank among both, and a selected key goes to
//      (keys above T before it) + min(keys equal to T before it, need), so
//      indices come out ascending and ties go to the lower index.
// Rows longer than 65536 tokens use the 8-bit streaming variant below.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kThreads = 1024;

// Phase marks for instrumented builds (nothing in the library build).
#ifndef DATTN_TOPK_MARK
#define DATTN_TOPK_MARK(i)
#endif
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 4096;
constexpr int kDigit = 12;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix sum over a block of NT threads; also returns the total
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* wave_tot,
                                                         uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const uint32_t v = lane < NW ? wave_tot[lane] : 0u;
    uint32_t vi = v;
#pragma unroll
    for (int d = 1; d < NW; d <<= 1) {
      const uint32_t y = __shfl_up(vi, d);
      if (lane >= d) vi += y;
    }
    if (lane < NW) wave_tot[lane] = vi - v;
    if (lane == NW - 1) wave_tot[NW] = vi;
  }
  __syncthreads();
  const uint32_t res = wave_tot[wave] + inc - x;
  total = wave_tot[NW];
  __syncthreads();
  return res;
}

template <int NT>
__device__ __forceinline__ uint32_t block_reduce_min_max(uint32_t mn, uint32_t mx, uint32_t* red,
                                                         uint32_t& out_max) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor(mn, d));
    mx = max(mx, (uint32_t)__shfl_xor(mx, d));
  }
  if (lane == 0) {
    red[wave] = mn;
    red[NW + wave] = mx;
  }
  __syncthreads();
  uint32_t a = 0xffffffffu, b = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a = min(a, red[w]);
    b = max(b, red[NW + w]);
  }
  __syncthreads();
  out_max = b;
  return a;
}

// Per-column ballot counts -> exclusive offsets: cnt[j][w] becomes the number
// of marked keys in columns < j plus those of waves < w in column j.
template <int NT, int KPT>
__device__ __forceinline__ void column_offsets(uint32_t (*cnt)[NT / 64], uint32_t* base) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  __syncthreads();
  for (int j = tid; j < KPT; j += NT) {
    uint32_t acc = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = cnt[j][w];
      cnt[j][w] = acc;
      acc += c;
    }
    base[j] = acc;
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of the column totals, 64 lanes over KPT columns
    constexpr int PER = (KPT + 63) / 64;
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int j = tid * PER + q;
      c[q] = j < KPT ? base[j] : 0u;
      sum += c[q];
    }
    uint32_t inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(inc, d);
      if (tid >= d) inc += y;
    }
    uint32_t acc = inc - sum;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int j = tid * PER + q;
      if (j < KPT) base[j] = acc;
      acc += c[q];
    }
  }
  __syncthreads();
}

// Keys resident on chip: columns [0, RK) in registers, [RK, RK + LK) in LDS
// (column c holds tokens c*NT .. c*NT + NT - 1, thread t owns token c*NT + t).
constexpr int kNT = 1024;
constexpr int kRK = 32;
constexpr int kLK = 32;
constexpr int kMaxCol = kRK + kLK;  // 65536 tokens
constexpr int kNW = kNT / 64;
constexpr size_t kResidentLds = (size_t)kLK * kNT * 4 + kBins * 4 + 2 * (size_t)kMaxCol * kNW * 4 +
                                2 * kMaxCol * 4 + (kNW + 1) * 4 + 2 * kNW * 4 + 16;

__global__ __launch_bounds__(kNT) void topk_kernel(const TopkArgs a) {
  constexpr int NT = kNT, NW = kNW, BPT = kBins / NT;
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* lds_keys = smem;                                     // [kLK][NT]
  uint32_t* hist = lds_keys + kLK * NT;                          // [kBins]
  uint32_t (*cnt_gt)[NW] = (uint32_t (*)[NW])(hist + kBins);     // [kMaxCol][NW]
  uint32_t (*cnt_eq)[NW] = cnt_gt + kMaxCol;                     // [kMaxCol][NW]
  uint32_t* base_gt = (uint32_t*)(cnt_eq + kMaxCol);             // [kMaxCol]
  uint32_t* base_eq = base_gt + kMaxCol;                         // [kMaxCol]
  uint32_t* wave_tot = base_eq + kMaxCol;                        // [NW + 1]
  uint32_t* red = wave_tot + NW + 1;                             // [2 NW]
  uint32_t* misc = red + 2 * NW;                                 // digit, need

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = a.seq_lens[b];
  const int K = a.k;
  const float* row = a.scores + (size_t)b * a.S_max;
  int32_t* out = a.idx + (size_t)b * K;

  if (L <= K) {
    for (int j = tid; j < K; j += NT) out[j] = j < L ? j : -1;
    return;
  }
  const int n_col = (L + NT - 1) / NT;
  DATTN_TOPK_MARK(0);

  // 1. one read of the row into order-preserving keys (0 past the row; real
  //    keys are >= 1: only an all-ones NaN pattern maps to 0, moved to 1),
  //    with the row's min and max
  uint32_t rk[kRK];
  uint32_t mn = 0xffffffffu, mx = 0u;
  {
    float x[kRK];
#pragma unroll
    for (int c = 0; c < kRK; ++c) x[c] = row[min(c * NT + tid, L - 1)];  // branch-free loads
#pragma unroll
    for (int c = 0; c < kRK; ++c) {
      rk[c] = c * NT + tid < L ? max(order_key(x[c]), 1u) : 0u;
      mn = min(mn, rk[c] ? rk[c] : 0xffffffffu);
      mx = max(mx, rk[c]);
    }
    constexpr int LB = (kLK + 1) / 2;  // two batches of loads for the LDS columns
    for (int c0 = kRK; c0 < n_col; c0 += LB) {
      float y[LB];
#pragma unroll
      for (int u = 0; u < LB; ++u) y[u] = row[min((c0 + u) * NT + tid, L - 1)];
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int c = c0 + u;
        const uint32_t k = c * NT + tid < L ? max(order_key(y[u]), 1u) : 0u;
        mn = min(mn, k ? k : 0xffffffffu);
        mx = max(mx, k);
        if (c < n_col) lds_keys[(c - kRK) * NT + tid] = k;
      }
    }
  }
  // visit every resident key of this thread: f(key, column); LDS columns go
  // in groups of 8 whose reads are issued together
  auto for_each = [&](auto&& f) {
#pragma unroll
    for (int c = 0; c < kRK; ++c)
      if (c < n_col) f(rk[c], c);
    for (int c0 = kRK; c0 < n_col; c0 += 8) {
      uint32_t y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = lds_keys[min(c0 + u - kRK, kLK - 1) * NT + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < n_col) f(y[u], c0 + u);
    }
  };
  DATTN_TOPK_MARK(1);
  uint32_t kmax;
  const uint32_t kmin = block_reduce_min_max<NT>(mn, mx, red, kmax);
  const uint32_t range = kmax - kmin;
  DATTN_TOPK_MARK(2);

  // 2. most significant digit first over v = key - kmin
  int hi_bit = range ? 32 - __clz(range) : 0;
  uint32_t prefix = 0, need = (uint32_t)K;
  while (hi_bit > 0) {
    const int width = hi_bit < kDigit ? hi_bit : kDigit;
    const int lo_bit = hi_bit - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    __syncthreads();
    for_each([&](uint32_t k, int) {
      const uint32_t v = k - kmin;
      if (k != 0u && (hi_bit >= 32 || (v >> hi_bit) == prefix)) atomicAdd(&hist[(v >> lo_bit) & dmask], 1u);
    });
    __syncthreads();
    // scan the bins from the top: thread t holds bins 4095-BPT*t downwards
    uint32_t cb[BPT], sum = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      cb[q] = hist[kBins - 1 - BPT * tid - q];
      sum += cb[q];
    }
    uint32_t tot;
    const uint32_t before = block_exclusive_scan<NT>(sum, wave_tot, tot);
    if (before < need && before + sum >= need) {
      uint32_t acc = before;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (acc + cb[q] >= need) {
          misc[0] = kBins - 1 - BPT * tid - q;
          misc[1] = need - acc;
          break;
        }
        acc += cb[q];
      }
    }
    __syncthreads();
    prefix = (prefix << width) | misc[0];
    need = misc[1];
    hi_bit = lo_bit;
    __syncthreads();
  }
  const uint32_t vT = prefix;  // the k-th largest key is kmin + vT
  DATTN_TOPK_MARK(3);

  // 3. ordered compaction.  A key above T is taken; of the keys equal to T
  //    the first `need` in index order are taken.  Its output position is
  //    (keys above T before it) + min(keys equal to T before it, need).
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  for_each([&](uint32_t k, int c) {
    const uint32_t v = k - kmin;
    const uint64_t mg = __ballot(k != 0u && v > vT);
    const uint64_t me = __ballot(k != 0u && v == vT);
    if (lane == 0) {
      cnt_gt[c][wave] = (uint32_t)__popcll(mg);
      cnt_eq[c][wave] = (uint32_t)__popcll(me);
    }
  });
  column_offsets<NT, kMaxCol>(cnt_gt, base_gt);
  column_offsets<NT, kMaxCol>(cnt_eq, base_eq);
  DATTN_TOPK_MARK(4);
  for_each([&](uint32_t k, int c) {
    const uint32_t v = k - kmin;
    const bool gt = k != 0u && v > vT, eq = k != 0u && v == vT;
    const uint64_t mg = __ballot(gt);
    const uint64_t me = __ballot(eq);
    const uint32_t r_gt = base_gt[c] + cnt_gt[c][wave] + (uint32_t)__popcll(mg & below);
    const uint32_t r_eq = base_eq[c] + cnt_eq[c][wave] + (uint32_t)__popcll(me & below);
    if (gt || (eq && r_eq < need)) {
      const uint32_t pos = r_gt + min(r_eq, need);
      if (pos < (uint32_t)K) out[pos] = c * NT + tid;  // always true when the select is right
    }
  });
  DATTN_TOPK_MARK(5);
}

// Streaming variant for rows longer than 1024 * 64 tokens: 8-bit digits over
// the raw key, scores re-read from memory every pass.
__global__ __launch_bounds__(kThreads) void topk_stream_kernel(const TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kWaves + 1];
  __shared__ uint32_t s_digit, s_need;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int L = a.seq_lens[b];
  const int K = a.k;
  const float* row = a.scores + (size_t)b * a.S_max;
  int32_t* out = a.idx + (size_t)b * K;

  if (L <= K) {
    for (int j = tid; j < K; j += kThreads) out[j] = j < L ? j : -1;
    return;
  }
  uint32_t prefix = 0, mask = 0, need = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < L; base += kThreads) {
      const int t = base + tid;
      bool act = false;
      uint32_t d = 0;
      if (t < L) {
        const uint32_t key = order_key(row[t]);
        act = (key & mask) == prefix;
        d = (key >> shift) & 255u;
      }
      const uint64_t actm = __ballot(act);
      if (actm == 0) continue;
      const int first = __ffsll((long long)actm) - 1;
      const uint32_t d0 = __shfl(d, first);
      const uint64_t same = __ballot(act && d == d0);
      if (same == actm) {
        if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
      } else if (act) {
        atomicAdd(&hist[d], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * tid - q];
        sum += c[q];
      }
      uint32_t inc = sum;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(inc, d);
        if (tid >= d) inc += y;
      }
      const uint32_t before = inc - sum;
      if (before < need && inc >= need) {
        uint32_t acc = before;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (acc + c[q] >= need) {
            s_digit = 255 - 4 * tid - q;
            s_need = need - acc;
            break;
          }
          acc += c[q];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    need = s_need;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int chunk = (L + kThreads - 1) / kThreads;
  const int lo = min(L, tid * chunk), hi = min(L, lo + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int t = lo; t < hi; ++t) {
    const uint32_t key = order_key(row[t]);
    n_gt += key > T;
    n_eq += key == T;
  }
  uint32_t tot;
  const uint32_t gt_before = block_exclusive_scan<kThreads>(n_gt, wave_tot, tot);
  const uint32_t eq_before = block_exclusive_scan<kThreads>(n_eq, wave_tot, tot);
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t eq_seen = eq_before;
  for (int t = lo; t < hi; ++t) {
    const uint32_t key = order_key(row[t]);
    bool take = key > T;
    if (key == T) take = eq_seen++ < need;
    if (take) {
      if (pos < (uint32_t)K) out[pos] = t;
      ++pos;
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.S_max <= kMaxCol * kNT) {
    static bool configured = false;
    if (!configured) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kResidentLds);
      if (e != hipSuccess) return e;
      configured = true;
    }
    topk_kernel<<<a.B, kNT, kResidentLds, s>>>(a);
  } else {
    topk_stream_kernel<<<a.B, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dattn
