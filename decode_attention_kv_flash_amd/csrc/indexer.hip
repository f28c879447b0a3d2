// DSA lightning-indexer scores: I[b,t] = sum_h w[b,h] * ReLU(q_i[b,h] . k_i[b,t]).
//
// ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
// Path": 64 indexer heads of 128 dims against a 128-value key cached per
// token, mixed by a per-head weight.)  The indexer reads every cached token,
// so this kernel is a stream over the key cache: 256 bytes per token, with
// the head contraction done on 32x32x16 bf16 MFMA (heads x tokens per
// instruction, K = 16 dims), fp32 accumulation.  Integer-valued inputs of
// modest size give exact scores.
//
// Work split: each wave takes 32-token steps of its workgroup's token range
// and keeps two of them in its own LDS buffers: a step's 8 KB of keys goes
// from HBM to LDS by eight direct-to-LDS copies of whole 1 KB runs (full
// cache lines), issued one step ahead.  The MFMA B fragment of lane l, k-step
// kk is token l % 32's dims 16 kk + 8 (l / 32) .. + 7: one 16-byte LDS read.
// Row r keeps its 16-byte chunk c at slot c ^ (r % 16), so the 16 rows a
// read instruction serves per pass hit 16 different bank groups.  The
// epilogue applies ReLU, the head weights, sums a lane's 32 heads in
// registers and the other 32 heads from lane l ^ 32.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kDi = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokWave = 32;   // tokens per wave step

constexpr int kRowBytes = kDi * 2;                 // 256
constexpr int kStepBytes = kTokWave * kRowBytes;    // 8 KB per wave step
constexpr int kCopies = kStepBytes / 1024;          // 8 wave-wide copies per step

template <int NMT>  // head tiles of 32: Hi = 32 * NMT
__global__ __launch_bounds__(kThreads) void indexer_kernel(const IndexerArgs a) {
  __shared__ __attribute__((aligned(16))) char kbuf[kWaves][2][kStepBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int lj = lane & 31;
  const int b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int Hi = 32 * NMT;

  // A fragments (heads x dims): lane holds head 32*mt + lj, dims 16*kk + 8*half + [0,8)
  uint4 qa[NMT][8];
  const uint16_t* qb = a.q + (size_t)b * Hi * kDi;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qa[mt][kk] = *(const uint4*)(qb + (size_t)(32 * mt + lj) * kDi + 16 * kk + 8 * half);
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

  const uint16_t* kbase = a.k + (size_t)b * a.S_max * kDi;
  float* out = a.scores + (size_t)b * a.S_max;
  // this workgroup's token range; its waves take its 32-token steps in turn
  const int t0 = blockIdx.x * a.tok_per_wg;
  const int t1 = min(a.S_max, t0 + a.tok_per_wg);
  const uint32_t my_lds = lds_address(&kbuf[wave][0][0]);

  // copy j fills slots 64 j + lane of a step buffer: row r = 4 j + lane / 16,
  // stored slot lane % 16, i.e. chunk (lane % 16) ^ (r % 16).  Rows past the
  // cache read its last row (finite data; their scores are not used).
  auto issue = [&](int tb, int buf) {
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      const int t = min(tb + r, a.S_max - 1);
      copy_to_lds(kbase + (size_t)t * kDi + 8 * c, my_lds + buf * kStepBytes + 1024 * j);
    }
  };

  int buf = 0;
  if (t0 + wave * kTokWave < t1) issue(t0 + wave * kTokWave, 0);
#pragma unroll 1
  for (int tb = t0 + wave * kTokWave; tb < t1; tb += kWaves * kTokWave) {
    if (tb + kWaves * kTokWave < t1) {
      issue(tb + kWaves * kTokWave, buf ^ 1);
      wait_vmcnt<kCopies>();  // this step's copies are in (the next step's may not be)
    } else {
      wait_vmcnt<0>();
    }
    const char* kb = &kbuf[wave][buf][0] + lj * kRowBytes;
    uint4 kv[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kv[kk] = *(const uint4*)(kb + 16 * ((2 * kk + half) ^ (lj & 15)));

    const int t = tb + lj;
    const bool valid = t < L;
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      f32x16_t acc = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qa[mt][kk]),
                                                      __builtin_bit_cast(bf16x8_t, kv[kk]),
                                                      acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) part = fmaf(wv[mt][v], fmaxf(acc[v], 0.f), part);
    }
    part += __shfl_xor(part, 32);
    if (half == 0 && t < a.S_max) out[t] = valid ? part : -__builtin_inff();
    buf ^= 1;
  }
}

// Workgroups resident per CU for this head count (at least 1), queried once.
template <int NMT>
int resident_per_cu() {
  static const int n = [] {
    int v = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, (const void*)indexer_kernel<NMT>, kThreads, 0) !=
            hipSuccess || v < 1)
      v = 1;
    return v;
  }();
  return n;
}

template <int NMT>
hipError_t launch_nmt(IndexerArgs a, hipStream_t s) {
  // one round of resident workgroups: the token ranges (whole 32-token steps)
  // are sized so that B x ranges just fills the CUs, with no partial second round
  const int64_t slots = (int64_t)device_cu_count() * resident_per_cu<NMT>();
  const int64_t tokens = (int64_t)a.B * a.S_max;
  int64_t per = (tokens + slots - 1) / slots;
  per = (per + kTokWave - 1) / kTokWave * kTokWave;
  if (per < kTokWave) per = kTokWave;
  a.tok_per_wg = (int32_t)per;
  dim3 grid((unsigned)((a.S_max + per - 1) / per), a.B), block(kThreads);
  indexer_kernel<NMT><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
  switch (a.Hi) {
    case 32: return launch_nmt<1>(a, s);
    case 64: return launch_nmt<2>(a, s);
    case 96: return launch_nmt<3>(a, s);
    case 128: return launch_nmt<4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dattn
