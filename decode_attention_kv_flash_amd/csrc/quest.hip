// Query-aware page selection (Quest): the two steps before the attention.
//
// ("Long context, KV eviction and sparse attention", "Sparse attention:
// choosing dynamically at every step": the cache is cut into pages of 16
// tokens; every page keeps the per-dimension minimum and maximum of its keys,
// and q . k over the page is bounded above by sum_d max(q_d kmin_d, q_d kmax_d);
// the pages with the largest bounds are attended, and the last, partial page
// always.  "Attention Optimizations", "Query-aware retrieval": a cheap
// per-page statistic decides which pages the query reads.)
//
// quest_minmax_kernel: one wave per (sequence, KV head, 16-token block); the
//   16 rows are read as in the split kernel (16 bytes per lane), reduced
//   across the lanes that hold the same columns, and written as the block's
//   [kmin | kmax] row in K's own type (exact: min and max pick input values).
//
// quest_bounds_kernel: the bound is a dense contraction.  With
//   q+ = max(q, 0) and q- = min(q, 0),
//     max(q_d kmin_d, q_d kmax_d) = q-_d kmin_d + q+_d kmax_d,
//   so upper[h, p] = [q- | q+]_h . [kmin | kmax]_p: a [heads x 2D] by
//   [2D x blocks] product, run on 16x16 MFMA tiles (16 heads x 16 blocks; a
//   group of G < 16 query heads leaves the other rows zero).  Each lane loads
//   16 contiguous bytes of one block's summary row per k-step, which is the
//   MFMA's B layout (lane l: column l % 16, k-slice l / 16), so the summary
//   goes from HBM to the matrix core without passing through LDS.  bf16 uses
//   16x16x32 bf16 MFMAs (products of bf16 values are exact in fp32), fp32 the
//   16x16x4 fp32 ones.  The kernel also writes each row's count of full
//   blocks, which the top-k select takes as the row length.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBlock = 16;   // tokens per summarised page
constexpr int kTiles = 2;    // 16-block tiles per wave in the bounds kernel

template <bool BF16, int D>
struct QShape {
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int VEC = 16 / ESZ;    // elements per 16-byte load
  static constexpr int LPR = D / VEC;     // lanes per row
  static constexpr int RPI = 64 / LPR;    // rows per wave load
  static constexpr int TPL = kBlock / RPI;  // rows per lane
  static constexpr int NS = 2 * D * ESZ / 64;  // 64-byte k-steps over a [kmin | kmax] row
};

__device__ __forceinline__ int full_blocks(const QuestArgs& a, int b) {
  const int L = max(a.seq_lens[b], 0);
  return min(L / kBlock, a.max_blocks);
}

// Address of row t of (sequence b, KV head kvh) in the K cache.
__device__ __forceinline__ const char* key_row(const QuestArgs& a, int b, int kvh, int t, int row_bytes) {
  size_t r;
  if (a.page_table) {
    const int phys = a.page_table[(size_t)b * a.max_pages + (t >> a.log2_page)];
    r = ((size_t)phys * a.Hkv + kvh) * a.page_size + (t & (a.page_size - 1));
  } else {
    r = ((size_t)b * a.Hkv + kvh) * a.page_size + t;  // contiguous: page_size = S_max
  }
  return (const char*)a.k + r * row_bytes;
}

__device__ __forceinline__ uint32_t min_bf16x2(uint32_t x, uint32_t y) {
  const float lo = fminf(bf16_lo(x), bf16_lo(y)), hi = fminf(bf16_hi(x), bf16_hi(y));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}
__device__ __forceinline__ uint32_t max_bf16x2(uint32_t x, uint32_t y) {
  const float lo = fmaxf(bf16_lo(x), bf16_lo(y)), hi = fmaxf(bf16_hi(x), bf16_hi(y));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

template <bool BF16>
__device__ __forceinline__ uint32_t min2(uint32_t x, uint32_t y) {
  if constexpr (BF16) return min_bf16x2(x, y);
  return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
}
template <bool BF16>
__device__ __forceinline__ uint32_t max2(uint32_t x, uint32_t y) {
  if constexpr (BF16) return max_bf16x2(x, y);
  return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void quest_minmax_kernel(const QuestArgs a) {
  using S = QShape<BF16, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk = (blockIdx.x + a.first_block / kWaves) * kWaves + wave;
  const int kvh = blockIdx.y, b = blockIdx.z;
  if (blk < a.first_block || blk >= full_blocks(a, b)) return;
  const int c = lane % S::LPR, r0 = lane / S::LPR;
  const char* base = key_row(a, b, kvh, blk * kBlock, D * S::ESZ);  // a block never straddles a page
  uint32_t mn[4], mx[4];
#pragma unroll
  for (int i = 0; i < S::TPL; ++i) {
    const uint4 x = *(const uint4*)(base + ((size_t)(r0 + i * S::RPI) * D + c * S::VEC) * S::ESZ);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mn[j] = i ? min2<BF16>(mn[j], w[j]) : w[j];
      mx[j] = i ? max2<BF16>(mx[j], w[j]) : w[j];
    }
  }
#pragma unroll
  for (int m = S::LPR; m < 64; m <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mn[j] = min2<BF16>(mn[j], (uint32_t)__shfl_xor((int)mn[j], m));
      mx[j] = max2<BF16>(mx[j], (uint32_t)__shfl_xor((int)mx[j], m));
    }
  }
  if (r0 == 0) {
    char* dst = (char*)a.kminmax + ((((size_t)b * a.Hkv + kvh) * a.max_blocks + blk) * 2 * D + c * S::VEC) * S::ESZ;
    *(uint4*)dst = make_uint4(mn[0], mn[1], mn[2], mn[3]);
    *(uint4*)(dst + D * S::ESZ) = make_uint4(mx[0], mx[1], mx[2], mx[3]);
  }
}

// The A operand for k-step s: the 16 bytes of [q- | q+] of head row `h` that
// pair with the summary bytes [64 s + 16 (lane / 16), +16) of a block row.
template <bool BF16, int D>
__device__ __forceinline__ uint4 signed_query(const char* qrow, bool valid, int s, int lane) {
  using S = QShape<BF16, D>;
  const int e = (64 * s + 16 * (lane >> 4)) / S::ESZ;  // element of the [kmin | kmax] row
  if (!valid) return make_uint4(0, 0, 0, 0);
  const bool upper_half = e >= D;  // kmax half pairs with q+, kmin half with q-
  const uint4 x = *(const uint4*)(qrow + (size_t)(upper_half ? e - D : e) * S::ESZ);
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (BF16) {
      // per bf16 half: keep it when its sign matches the half, else zero
      const uint32_t neg = ((w[j] >> 15) & 1u) * 0x0000ffffu | (w[j] >> 31) * 0xffff0000u;
      w[j] &= upper_half ? ~neg : neg;
    } else {
      const float f = __uint_as_float(w[j]);
      w[j] = __float_as_uint(upper_half ? fmaxf(f, 0.f) : fminf(f, 0.f));
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_step(const uint4& qa, const uint4& kb, f32x4_t acc) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa),
                                                   __builtin_bit_cast(bf16x8_t, kb), acc, 0, 0, 0);
  } else {
    // four k = 4 products, element 4 (lane / 16) + j of the 16 bytes' k-slice
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qa.x), __uint_as_float(kb.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qa.y), __uint_as_float(kb.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qa.z), __uint_as_float(kb.z), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qa.w), __uint_as_float(kb.w), acc, 0, 0, 0);
  }
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void quest_bounds_kernel(const QuestArgs a) {
  using S = QShape<BF16, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int head_tiles = (a.G + 15) / 16;
  const int kvh = blockIdx.y / head_tiles, ht = blockIdx.y % head_tiles;
  const int b = blockIdx.z;
  const int n_full = full_blocks(a, b);
  const int hq0 = kvh * a.G + ht * 16;         // first query head of this tile
  const int nh = min(16, a.G - ht * 16);       // heads in this tile
  if (blockIdx.x == 0 && wave == 0 && lane < nh) a.n_full[(size_t)b * a.Hq + hq0 + lane] = n_full;
  const int blk0 = (blockIdx.x * kWaves + wave) * kTiles * 16;
  if (blk0 >= n_full) return;

  const int hrow = lane & 15;
  const char* qrow = (const char*)a.q + ((size_t)b * a.Hq + hq0 + min(hrow, nh - 1)) * D * S::ESZ;
  uint4 qa[S::NS];
#pragma unroll
  for (int s = 0; s < S::NS; ++s) qa[s] = signed_query<BF16, D>(qrow, hrow < nh, s, lane);

  const char* sum_base = (const char*)a.kminmax + ((size_t)b * a.Hkv + kvh) * a.max_blocks * 2 * D * S::ESZ;
  uint4 kb[kTiles][S::NS];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int blk = min(blk0 + 16 * t + (lane & 15), n_full - 1);  // blocks past the row re-read its last
    const char* row = sum_base + (size_t)blk * 2 * D * S::ESZ + 16 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < S::NS; ++s) kb[t][s] = *(const uint4*)(row + 64 * s);
  }
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S::NS; ++s) acc = mfma_step<BF16>(qa[s], kb[t][s], acc);
    const int blk = blk0 + 16 * t + (lane & 15);
    if (blk < n_full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * (lane >> 4) + i;  // the MFMA's output row
        if (h < nh) a.upper[((size_t)b * a.Hq + hq0 + h) * a.max_blocks + blk] = acc[i];
      }
    }
  }
}

// One workgroup per (sequence, KV head): the blocks the group's G query
// heads chose become one bitmap per head in LDS.  Thread t owns word t of
// their union and an exclusive prefix sum over the words' populations gives
// each word's first position; then every thread places blocks of its own
// (blk = t, t + 256, ...) at that position plus the union bits below it in
// its word, so the union comes out ascending, each entry carrying the heads
// that chose the block.
__global__ __launch_bounds__(kThreads) void quest_union_kernel(const QuestUnionArgs a) {
  constexpr int kWords = kQuestUnionMaxBlocks / 32;
  static_assert(kWords == kThreads, "one bitmap word per thread");
  __shared__ uint32_t bm[8][kWords];
  __shared__ uint32_t uw[kWords], first[kWords];
  __shared__ uint32_t wave_sum[kWaves];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int L = max(a.seq_lens[b], 0);
  const int n_full = min(L / kBlock, a.max_blocks);
  const int kept = min(a.budget, n_full);
  const int words = (n_full + 31) / 32;
  for (int h = 0; h < a.G; ++h) bm[h][t] = 0u;
  __syncthreads();
  for (int i = t; i < a.G * kept; i += kThreads) {
    const int h = i / kept, j = i - h * kept;
    const int blk = a.sel[((size_t)b * a.Hq + kvh * a.G + h) * a.budget + j];
    if (blk >= 0 && blk < n_full) atomicOr(&bm[h][blk >> 5], 1u << (blk & 31));
  }
  __syncthreads();
  uint32_t u = 0u;
  for (int h = 0; h < a.G; ++h) u |= bm[h][t];
  const uint32_t cnt = __popc(u);
  uint32_t inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_sum[wave] = inc;
  __syncthreads();
  uint32_t before = inc - cnt;
  for (int w = 0; w < wave; ++w) before += wave_sum[w];
  uw[t] = u;
  first[t] = before;
  if (t == kThreads - 1) a.count[(size_t)b * a.Hkv + kvh] = min((int)(before + cnt), a.cap);
  __syncthreads();
  int32_t* out = a.list + ((size_t)b * a.Hkv + kvh) * a.cap;
  for (int blk = t; blk < 32 * words; blk += kThreads) {
    const int w = blk >> 5, j = blk & 31;
    const uint32_t x = uw[w];
    if (!((x >> j) & 1u)) continue;
    const uint32_t k = first[w] + __popc(x & ((1u << j) - 1u));
    uint32_t heads = 0u;
    for (int h = 0; h < a.G; ++h) heads |= ((bm[h][w] >> j) & 1u) << h;
    if (k < (uint32_t)a.cap) out[k] = blk | (int32_t)(heads << 24);
  }
}

template <bool BF16, int D>
hipError_t minmax_d(const QuestArgs& a, hipStream_t s) {
  const int wgs = (a.max_blocks + kWaves - 1) / kWaves - a.first_block / kWaves;
  if (wgs <= 0) return hipSuccess;
  dim3 grid(wgs, a.Hkv, a.B);
  launch_kernel(quest_minmax_kernel<BF16, D>, grid, kThreads, s, a);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t bounds_d(const QuestArgs& a, hipStream_t s) {
  const int per_wg = kWaves * kTiles * 16;
  dim3 grid((a.max_blocks + per_wg - 1) / per_wg, a.Hkv * ((a.G + 15) / 16), a.B);
  launch_kernel(quest_bounds_kernel<BF16, D>, grid, kThreads, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quest_minmax(const QuestArgs& a, hipStream_t s) {
  if (a.bf16) return a.D == 64 ? minmax_d<true, 64>(a, s) : minmax_d<true, 128>(a, s);
  return a.D == 64 ? minmax_d<false, 64>(a, s) : minmax_d<false, 128>(a, s);
}

hipError_t launch_quest_union(const QuestUnionArgs& a, hipStream_t s) {
  if (a.G > 8 || a.max_blocks > kQuestUnionMaxBlocks) return hipErrorInvalidValue;
  launch_kernel(quest_union_kernel, dim3(a.Hkv, a.B), kThreads, s, a);
  return hipGetLastError();
}

hipError_t launch_quest_bounds(const QuestArgs& a, hipStream_t s) {
  if (a.bf16) return a.D == 64 ? bounds_d<true, 64>(a, s) : bounds_d<true, 128>(a, s);
  return a.D == 64 ? bounds_d<false, 64>(a, s) : bounds_d<false, 128>(a, s);
}

}  // namespace dattn
