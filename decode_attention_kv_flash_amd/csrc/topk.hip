// Top-k token selection over fp32 scores: the k largest of each row, ties to
// the lower token index, written in ascending index order, -1 padded.
//
// ("Attention Optimizations", "Computation Path": indices = topk(I, 2048);
// "Caveats": a top-k over the whole context is expensive, so it is a radix
// select, not a sort.)  One workgroup per row:
//   1. scores become order-preserving unsigned keys (-0.0 folded onto +0.0);
//   2. four passes of an 8-bit radix select find the k-th largest key T and
//      how many keys equal to T are still needed (`need`): each pass builds a
//      256-bin histogram in LDS of the keys that match the digits fixed so
//      far -- a wave whose keys share one digit adds its count with a single
//      atomic -- and one wave scans it from the top;
//   3. an ordered compaction: each thread owns a contiguous range of indices,
//      counts keys > T and keys == T in it, two block-wide exclusive scans
//      give each thread its output offset and how many equal keys precede it,
//      and the thread writes its selected indices in increasing order.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix sum over the block; also returns the block total
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* wave_tot,
                                                         uint32_t& total) {
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
    uint32_t v = lane < kWaves ? wave_tot[lane] : 0u;
    uint32_t vi = v;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const uint32_t y = __shfl_up(vi, d);
      if (lane >= d) vi += y;
    }
    if (lane < kWaves) wave_tot[lane] = vi - v;  // exclusive
    if (lane == kWaves - 1) wave_tot[kWaves] = vi;
  }
  __syncthreads();
  const uint32_t res = wave_tot[wave] + inc - x;
  total = wave_tot[kWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const TopkArgs a) {
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
      // bins 255..0: lane j holds bins 255-4j .. 252-4j
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
      uint32_t before = inc - sum;  // keys in higher bins than this lane's
      // the digit is in the first lane whose cumulative count reaches `need`
      const bool here = before < need && inc >= need;
      if (here) {
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

  // ordered compaction over contiguous per-thread ranges
  const int chunk = (L + kThreads - 1) / kThreads;
  const int lo = min(L, tid * chunk), hi = min(L, lo + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int t = lo; t < hi; ++t) {
    const uint32_t key = order_key(row[t]);
    n_gt += key > T;
    n_eq += key == T;
  }
  uint32_t tot;
  const uint32_t gt_before = block_exclusive_scan(n_gt, wave_tot, tot);
  const uint32_t eq_before = block_exclusive_scan(n_eq, wave_tot, tot);
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t eq_seen = eq_before;
  for (int t = lo; t < hi; ++t) {
    const uint32_t key = order_key(row[t]);
    bool take = key > T;
    if (key == T) take = eq_seen++ < need;
    if (take) {
      if (pos < (uint32_t)K) out[pos] = t;  // always true when the select is right
      ++pos;
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  topk_kernel<<<a.B, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dattn
