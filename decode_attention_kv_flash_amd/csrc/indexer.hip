// DSA lightning-indexer scores: I[b,t] = sum_h w[b,h] * ReLU(q_i[b,h] . k_i[b,t]).
//
// ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
// Path": 64 indexer heads of 128 dims against a 128-value key cached per
// token, mixed by a per-head weight.)  The indexer reads every cached token,
// so this kernel is a stream over the key cache: 256 bytes per token in
// bf16, 128 in fp8 e4m3 (the precision the pages give the lightning indexer:
// "Long context ...", "Sparse attention: choosing dynamically at every
// step"), with the head contraction on 32x32x16 MFMAs of either type (heads x
// tokens per instruction, K = 16 dims), fp32 accumulation.  Integer-valued
// inputs of modest size give exact scores (in fp8 e4m3, integers up to 16 are
// exact).
//
// Work split: each wave takes steps of its workgroup's token range (32
// tokens in bf16, 64 in fp8: 8 KB either way) and keeps three of them in its
// own LDS buffers: a step's keys go
// from HBM to LDS by direct-to-LDS copies of whole 1 KB runs (full cache
// lines), issued two steps ahead.  The MFMA B fragments of lane l are token
// l % 32's dims (bf16: 16 kk + 8 (l / 32) .. + 7, one 16-byte LDS read per
// k-step; fp8: 64 (l / 32) + 8 kk .. + 7, four 16-byte reads for all eight).
// Rows keep their 16-byte chunks permuted by a row key (slot_key), so the
// rows a read instruction serves per pass hit different bank groups.  The
// epilogue applies ReLU, the head weights, sums a lane's 32 heads in
// registers and the other 32 heads from lane l ^ 32.  When a workgroup's
// token range is one chunk of the top-k select, it also counts its scores'
// top key bytes into the select's first-level histogram (one launch fewer).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kDi = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokMma = 32;    // tokens per MFMA (the B operand's columns)
// 8 KB step buffers per wave: two steps in flight while one is computed.
// (96 KB of LDS per workgroup, one workgroup per CU; measured against two
// buffers at two workgroups per CU and four or five at one: 24.1 us against
// 25.9, 24.3 and 25.1 us for 8 x 65536 bf16 keys.)
constexpr int kBufs = 3;

template <bool FP8>
struct IdxShape {
  static constexpr int kRowBytes = FP8 ? kDi : 2 * kDi;       // 128 or 256
  static constexpr int kChunks = kRowBytes / 16;              // 16-byte chunks per row
  static constexpr int kTokStep = FP8 ? 64 : 32;               // tokens per wave step
  static constexpr int kStepBytes = kTokStep * kRowBytes;      // 8 KB per wave step
  static constexpr int kCopies = kStepBytes / 1024;            // wave-wide 1 KB copies per step
};

// Stored slot of chunk c of step row r: c ^ (r % 16) for the 16-chunk bf16
// rows; c ^ ((r / 2) % 8) for the 8-chunk fp8 rows (two rows share a 256-byte
// bank window, so rows of equal parity take distinct slots).
template <bool FP8>
__device__ __forceinline__ int slot_key(int r) {
  return FP8 ? (r >> 1) & 7 : r & 15;
}

// HI = 32 * NMT heads.  bf16: 32x32x16 bf16 MFMAs, lane (head or token l % 32,
// half l / 32) holds dims 16 kk + 8 half + [0, 8) of k-step kk.  fp8 e4m3:
// 32x32x16 fp8 MFMAs, the lane holds dims 64 half + 8 kk + [0, 8) (one
// 64-byte run of the row); both operands use the same dims at the same
// (lane, k-step, slot), so the contraction is the plain dot product.
// Wait until at most `later` x COPIES vector-memory operations of this wave
// are outstanding (later in [0, AHEAD]).
template <int AHEAD, int COPIES>
__device__ __forceinline__ void wait_copies_after(int later) {
  static_assert(AHEAD * COPIES < 64, "vmcnt range");
  if constexpr (AHEAD >= 4) if (later == 4) { wait_vmcnt<4 * COPIES>(); return; }
  if constexpr (AHEAD >= 3) if (later == 3) { wait_vmcnt<3 * COPIES>(); return; }
  if constexpr (AHEAD >= 2) if (later == 2) { wait_vmcnt<2 * COPIES>(); return; }
  if constexpr (AHEAD >= 1) if (later == 1) { wait_vmcnt<COPIES>(); return; }
  wait_vmcnt<0>();
}

template <int NMT, bool FP8>
__global__ __launch_bounds__(kThreads) void indexer_kernel(const IndexerArgs a) {
  using S = IdxShape<FP8>;
  __shared__ __attribute__((aligned(16))) char kbuf[kWaves][kBufs][S::kStepBytes];
  __shared__ uint32_t hist[256];  // top key byte of this range's valid scores (a.hist0 only)
  if (a.hist0) {
    hist[threadIdx.x] = 0u;
    barrier_in_flight<63>();  // LDS only: nothing else is waited for
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int lj = lane & 31;
  const int b = blockIdx.y;
  const int L = min(max(a.seq_lens[b], 0), a.S_max);  // a caller contract, clamped to the cache
  const int Hi = 32 * NMT;

  // A fragments (heads x dims): lane holds head 32*mt + lj
  typedef typename std::conditional<FP8, uint2, uint4>::type frag_t;
  frag_t qa[NMT][8];
  const char* qb = (const char*)a.q + (size_t)b * Hi * S::kRowBytes;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const char* row = qb + (size_t)(32 * mt + lj) * S::kRowBytes;
      if constexpr (FP8) qa[mt][kk] = *(const uint2*)(row + 64 * half + 8 * kk);
      else qa[mt][kk] = *(const uint4*)(row + 2 * (16 * kk + 8 * half));
    }
  }
  // head weights of the 16 accumulator rows this lane holds per head tile:
  // row(v) = 8*(v/4) + 4*half + (v%4)
  float wv[NMT][16];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      wv[mt][v] = a.w[(size_t)b * Hi + 32 * mt + 8 * (v / 4) + 4 * half + (v % 4)];
  }

  const char* kbase = (const char*)a.k + (size_t)b * a.S_max * S::kRowBytes;
  float* out = a.scores + (size_t)b * a.S_max;
  // this workgroup's token range (whole steps); its waves take its steps in turn
  const int t0 = blockIdx.x * a.tok_per_wg;
  const int t1 = min(a.S_max, t0 + a.tok_per_wg);
  const uint32_t my_lds = lds_address(&kbuf[wave][0][0]);

  // copy j fills slots 64 j + lane of a step buffer: row r = 64 j / chunks +
  // lane / chunks, stored slot lane % chunks, which holds chunk
  // slot ^ key(r).  Rows past the cache read its last row (finite data;
  // their scores are not used).
  auto issue = [&](int tb, int buf) {
#pragma unroll
    for (int j = 0; j < S::kCopies; ++j) {
      const int r = (64 / S::kChunks) * j + lane / S::kChunks;
      const int c = (lane % S::kChunks) ^ slot_key<FP8>(r);
      const int t = min(tb + r, a.S_max - 1);
      copy_to_lds(kbase + (size_t)t * S::kRowBytes + 16 * c, my_lds + buf * S::kStepBytes + 1024 * j);
    }
  };

  // The wave's steps j = 0 .. n_steps - 1 start at token t0 + (wave + kWaves j)
  // kStep; step j lives in buffer j % kBufs and is requested kAhead steps
  // before it is used.  Before using step j the wave waits until only the
  // copies of the steps requested after it (at most kAhead) are in flight;
  // the score stores it has issued meanwhile are not counted, which only
  // makes the wait stricter.
  constexpr int kStep = S::kTokStep;
  constexpr int kAhead = kBufs - 1;
  const int first = t0 + wave * kStep;
  const int n_steps = first < t1 ? (t1 - first + kWaves * kStep - 1) / (kWaves * kStep) : 0;
#pragma unroll
  for (int j = 0; j < kAhead; ++j)
    if (j < n_steps) issue(first + j * kWaves * kStep, j);
  int buf = 0, nbuf = kAhead;  // buffer of step j, and of step j + kAhead
#pragma unroll 1
  for (int j = 0; j < n_steps; ++j) {
    const int tb = first + j * kWaves * kStep;
    if (j + kAhead < n_steps) issue(tb + kAhead * kWaves * kStep, nbuf);
    const int later = min(kAhead, n_steps - 1 - j);  // steps requested after this one
    wait_copies_after<kAhead, S::kCopies>(later);
#pragma unroll
    for (int sub = 0; sub < kStep / kTokMma; ++sub) {
    const char* kb = &kbuf[wave][buf][0] + (kTokMma * sub + lj) * S::kRowBytes;
    frag_t kv[8];
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 x = *(const uint4*)(kb + 16 * ((4 * half + c) ^ slot_key<true>(lj)));
        kv[2 * c] = make_uint2(x.x, x.y);
        kv[2 * c + 1] = make_uint2(x.z, x.w);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) kv[kk] = *(const uint4*)(kb + 16 * ((2 * kk + half) ^ slot_key<false>(lj)));
    }

    const int t = tb + kTokMma * sub + lj;
    const bool valid = t < L;
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      f32x16_t acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        if constexpr (FP8)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(__builtin_bit_cast(long, qa[mt][kk]),
                                                           __builtin_bit_cast(long, kv[kk]), acc, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qa[mt][kk]),
                                                        __builtin_bit_cast(bf16x8_t, kv[kk]), acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) part = fmaf(wv[mt][v], fmaxf(acc[v], 0.f), part);
    }
    part += __shfl_xor(part, 32);
    if (half == 0 && t < a.S_max) out[t] = valid ? part : -__builtin_inff();
    if (a.hist0 && half == 0 && valid) atomicAdd(&hist[order_key(part) >> 24], 1u);
    }
    buf = buf == kBufs - 1 ? 0 : buf + 1;
    nbuf = nbuf == kBufs - 1 ? 0 : nbuf + 1;
  }
  if (a.hist0) {
    barrier_in_flight<63>();  // every wave's counts are in LDS
    a.hist0[(size_t)b * a.hist_row_words + (size_t)blockIdx.x * 256 + threadIdx.x] = hist[threadIdx.x];
  }
}

// Workgroups resident per CU for this head count (at least 1), queried once.
template <int NMT, bool FP8>
int resident_per_cu() {
  static const int n = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, (const void*)indexer_kernel<NMT, FP8>, kThreads, 0) !=
            hipSuccess || v < 1)
      v = 1;
    return v;
  }();
  return n;
}

template <int NMT, bool FP8>
hipError_t launch_nmt(IndexerArgs& a, hipStream_t s) {
  // one round of resident workgroups: at most slots / B token ranges (whole
  // wave steps) per row, so that B x ranges never spills into a second round
  // (sized from B x S_max / slots rounded up, 6 rows of 65536 tokens made
  // 258 workgroups for 256 slots: 48.8 us for the indexer and top-k against
  // 42.5 us for 8 rows)
  const int64_t slots = (int64_t)device_cu_count() * resident_per_cu<NMT, FP8>();
  constexpr int kStep = IdxShape<FP8>::kTokStep;
  const int64_t ranges = std::max<int64_t>(1, slots / a.B);
  int64_t per = (a.S_max + ranges - 1) / ranges;
  per = (per + kStep - 1) / kStep * kStep;
  if (per < kStep) per = kStep;
  a.tok_per_wg = (int32_t)per;
  // the select's first level comes along only when the ranges are its chunks
  if (per != kTopkChunk || a.S_max <= kTopkChunk) a.hist0 = nullptr;
  dim3 grid((unsigned)((a.S_max + per - 1) / per), a.B), block(kThreads);
  launch_kernel(indexer_kernel<NMT, FP8>, grid, block, s, a);
  return hipGetLastError();
}

template <bool FP8>
hipError_t launch_type(IndexerArgs& a, hipStream_t s) {
  switch (a.Hi) {
    case 32: return launch_nmt<1, FP8>(a, s);
    case 64: return launch_nmt<2, FP8>(a, s);
    case 96: return launch_nmt<3, FP8>(a, s);
    case 128: return launch_nmt<4, FP8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_indexer(IndexerArgs& a, hipStream_t s) {
  return a.fp8 ? launch_type<true>(a, s) : launch_type<false>(a, s);
}

}  // namespace dattn
