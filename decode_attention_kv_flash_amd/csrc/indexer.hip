// DSA lightning-indexer scores: I[b,t] = sum_h w[b,h] * ReLU(q_i[b,h] . k_i[b,t]).
//
// ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
// Path": 64 indexer heads of 128 dims against a 128-value key cached per
// token, mixed by a per-head weight.)  The indexer reads every cached token,
// so this kernel is a stream over the key cache: 256 bytes per token, with
// the 64-head contraction done on 32x32x16 bf16 MFMA (heads x tokens per
// instruction, K = 16 dims), fp32 accumulation.  Integer-valued inputs of
// modest size give exact scores.
//
// Work split: a wave takes 32 tokens per step; lane l streams 128 contiguous
// bytes (64 dims) of token (l % 32)'s key -- dims [64*(l/32), 64*(l/32)+64) --
// which is its B fragment for eight k-steps when the dot product's K index is
// permuted the same way for the query fragments (the sum does not depend on
// the order of the dims).  The epilogue applies ReLU, the head weights, sums
// a lane's 32 heads in registers and the other 32 heads from lane l ^ 32.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kDi = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTokWave = 32;   // tokens per wave step
constexpr int kStepsPerWave = 4;
constexpr int kTokWG = kTokWave * kWaves * kStepsPerWave;  // 512

template <int NMT>  // head tiles of 32: Hi = 32 * NMT
__global__ __launch_bounds__(kThreads) void indexer_kernel(const IndexerArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int lj = lane & 31;
  const int b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int Hi = 32 * NMT;

  // A fragments (heads x dims): lane holds head 32*mt + lj, dims 64*half + 8*kk + [0,8)
  uint4 qa[NMT][8];
  const uint16_t* qb = a.q + (size_t)b * Hi * kDi;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qa[mt][kk] = *(const uint4*)(qb + (size_t)(32 * mt + lj) * kDi + 64 * half + 8 * kk);
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
  const int t0 = blockIdx.x * kTokWG;

#pragma unroll 1
  for (int st = 0; st < kStepsPerWave; ++st) {
    const int tb = t0 + (st * kWaves + wave) * kTokWave;
    if (tb >= a.S_max) break;
    const int t = tb + lj;
    const bool valid = t < L;
    uint4 kv[8];
    const uint16_t* src = kbase + (size_t)t * kDi + 64 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      kv[kk] = valid ? *(const uint4*)(src + 8 * kk) : make_uint4(0u, 0u, 0u, 0u);

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
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
  dim3 grid((a.S_max + kTokWG - 1) / kTokWG, a.B), block(kThreads);
  switch (a.Hi) {
    case 32: indexer_kernel<1><<<grid, block, 0, s>>>(a); break;
    case 64: indexer_kernel<2><<<grid, block, 0, s>>>(a); break;
    case 96: indexer_kernel<3><<<grid, block, 0, s>>>(a); break;
    case 128: indexer_kernel<4><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dattn
