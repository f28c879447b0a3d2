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
// Work is cut into 16-token blocks aligned to the page (a paged cache with
// page_size a multiple of 16, or a contiguous cache): the page of a block is
// one wave-uniform table lookup, and a lane's addresses are fixed offsets
// from it.  The set's partial first and last blocks are masked per token.
// Inside a workgroup each wave streams its own blocks:
//   * eight lanes cover a 128-byte segment of a token row (16 bytes each), so
//     one wave load instruction reads eight full 128-byte lines, and a lane
//     holds D*size/128 segments of two tokens per block;
//   * scores are lane-partial dot products (v_dot2_f32_bf16 for bf16: the
//     bf16 products are exact in fp32) summed over the 8 lanes with DPP;
//   * the softmax is the online one ("All the attentions", section 1: a
//     running maximum and running sum, earlier partials rescaled), kept per
//     token row of the wave; the reference maximum only moves when the new
//     maximum exceeds it by more than 2^8, which bounds every exponential by
//     2^8 and makes rescaling rare without changing the result;
//   * P.V: for bf16 the two tokens' probabilities are rounded to bf16 and
//     paired with the two tokens' values in one v_dot2_f32_bf16 per output
//     (fp32 accumulation); for fp32 inputs it is plain fp32 FMA.
// A split's result is (o / l, log2-sum-exp); lse_combine merges the splits
// (lse = max + log2 sum 2^(lse_j - max), o = sum 2^(lse_j - lse) o_j).
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 16;     // tokens per wave step
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
#ifndef DATTN_GQA_UNROLL
#define DATTN_GQA_UNROLL 1
#endif
constexpr int kUnroll = DATTN_GQA_UNROLL;  // blocks whose loads a wave issues together

template <bool BF16, int D>
struct GqaShape {
  static constexpr int ESZ = BF16 ? 2 : 4;   // bytes per element
  static constexpr int VEC = 16 / ESZ;       // elements per 16-byte piece
  static constexpr int SEG = 128 / ESZ;      // elements per 128-byte segment
  static constexpr int NH = D / SEG;         // 128-byte segments per row
  static constexpr int DL = VEC * NH;        // dims a lane holds per token
  static_assert(NH >= 1 && D % SEG == 0, "row split");
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

__device__ __forceinline__ uint32_t u4(const uint4& x, int w) {
  return w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
}

// PAGED_FAST: paged with page_size % 16 == 0, or contiguous (one lookup per
// block); otherwise every token resolves its own page.
template <bool BF16, int D, int G, bool PAGED_FAST>
__global__ __launch_bounds__(kThreads) void gqa_split_kernel(const GqaArgs a) {
  using S = GqaShape<BF16, D>;
  constexpr int VEC = S::VEC, SEG = S::SEG, NH = S::NH, DL = S::DL;
  const float NEG_INF = -__builtin_inff();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 3;   // token row within an 8-row load
  const int c = lane & 7;    // 16-byte column within a 128-byte segment
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;

  // Token set [0, s_cnt) u [w_start, L) as 16-token blocks: sink blocks
  // first, then the window's blocks (aligned down to 16).
  const int L = a.seq_lens[b];
  int s_cnt = 0, w_start = 0;
  if (a.window > 0 && a.window < L) {
    w_start = L - a.window;
    s_cnt = min(a.n_sink, w_start);
  }
  const int n_sb = (s_cnt + kStep - 1) / kStep;
  const int wb0 = w_start / kStep;
  const int n_wb = L > 0 ? (L + kStep - 1) / kStep - wb0 : 0;
  const int n_blocks = n_sb + n_wb;
  const int per = (n_blocks + a.num_splits - 1) / a.num_splits;
  const int blk_begin = min(n_blocks, split * per);
  const int blk_end = min(n_blocks, blk_begin + per);

  // This lane's pieces of the G query rows: dims hh*SEG + c*VEC + [0, VEC).
  uint4 qv[G][NH];
  {
    const char* qb = (const char*)a.q + ((size_t)(b * a.Hq + kvh * G) * D + c * VEC) * S::ESZ;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        qv[h][hh] = *(const uint4*)(qb + ((size_t)h * D + hh * SEG) * S::ESZ);
  }

  float m[G], l[G], o[G][DL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = NEG_INF;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[h][e] = 0.f;
  }

  const size_t head_stride = (size_t)a.page_size * D;
  const size_t page_stride = (size_t)a.Hkv * head_stride;
  const char* kb = (const char*)a.k;
  const char* vb = (const char*)a.v;
  const int32_t* pt = a.page_table ? a.page_table + (size_t)b * a.max_pages : nullptr;
  const size_t contig_base = ((size_t)b * a.Hkv + kvh) * head_stride;
  const size_t lane_off = (size_t)c * VEC * S::ESZ;

  auto block_start = [&](int blk) {
    return blk < n_sb ? blk * kStep : (wb0 + blk - n_sb) * kStep;
  };
  // physical page of the next block, loaded one block ahead
  int phys_next = 0;
  if (PAGED_FAST && pt && blk_begin + wave < blk_end)
    phys_next = pt[block_start(blk_begin + wave) >> a.log2_page];

  for (int blk0 = blk_begin + wave; blk0 < blk_end; blk0 += kWaves * kUnroll) {
    // issue the loads of kUnroll blocks of this wave, then compute them
    uint4 kr[kUnroll][2][NH], vr[kUnroll][2][NH];
    bool valid[kUnroll][2];
#pragma unroll
    for (int x = 0; x < kUnroll; ++x) {
      const int blk = blk0 + x * kWaves;
      const bool live = blk < blk_end;
      const bool sink = blk < n_sb;
      const int t0 = block_start(blk);
      const int lo = sink ? 0 : w_start;
      const int hi = live ? (sink ? s_cnt : L) : 0;
      size_t base_fast = 0;
      if constexpr (PAGED_FAST) {
        if (pt) {
          const int phys = phys_next;
          if (blk + kWaves < blk_end) phys_next = pt[block_start(blk + kWaves) >> a.log2_page];
          base_fast = (size_t)phys * page_stride + (size_t)kvh * head_stride +
                      (size_t)(t0 & (a.page_size - 1)) * D;
        } else {
          base_fast = contig_base + (size_t)t0 * D;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = t0 + 8 * u + r;
        valid[x][u] = t >= lo && t < hi;
        size_t off;
        if constexpr (PAGED_FAST) {
          off = (base_fast + (size_t)(8 * u + r) * D) * S::ESZ + lane_off;
        } else {
          const int phys = valid[x][u] ? pt[t >> a.log2_page] : 0;
          off = ((size_t)phys * page_stride + (size_t)kvh * head_stride +
                 (size_t)(t & (a.page_size - 1)) * D) * S::ESZ + lane_off;
        }
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          if (valid[x][u]) {
            kr[x][u][hh] = load_stream(kb + off + hh * 128);
            vr[x][u][hh] = load_stream(vb + off + hh * 128);
          } else {
            kr[x][u][hh] = make_uint4(0u, 0u, 0u, 0u);
            vr[x][u][hh] = make_uint4(0u, 0u, 0u, 0u);
          }
        }
      }
    }

#pragma unroll
    for (int x = 0; x < kUnroll; ++x) {
    // scores (log2 units) of the lane's two tokens
    float s[2][G];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          if constexpr (BF16) {
            acc = dot2_bf16(kr[x][u][hh].x, qv[h][hh].x, acc);
            acc = dot2_bf16(kr[x][u][hh].y, qv[h][hh].y, acc);
            acc = dot2_bf16(kr[x][u][hh].z, qv[h][hh].z, acc);
            acc = dot2_bf16(kr[x][u][hh].w, qv[h][hh].w, acc);
          } else {
            acc = fmaf(__uint_as_float(kr[x][u][hh].x), __uint_as_float(qv[h][hh].x), acc);
            acc = fmaf(__uint_as_float(kr[x][u][hh].y), __uint_as_float(qv[h][hh].y), acc);
            acc = fmaf(__uint_as_float(kr[x][u][hh].z), __uint_as_float(qv[h][hh].z), acc);
            acc = fmaf(__uint_as_float(kr[x][u][hh].w), __uint_as_float(qv[h][hh].w), acc);
          }
        }
        acc = group_sum<8>(acc) * a.scale_log2;
        s[u][h] = valid[x][u] ? acc : NEG_INF;
      }
    }

    // online softmax with a lazily moved reference maximum
    float p[2][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = fmaxf(s[0][h], s[1][h]);
      if (mx > m[h] + kTau) {
        const float alpha = fast_exp2(m[h] - mx);  // 0 when m was -inf
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < DL; ++e) o[h][e] *= alpha;
        m[h] = mx;
      }
      const float mu = m[h] == NEG_INF ? 0.f : m[h];
      p[0][h] = fast_exp2(s[0][h] - mu);
      p[1][h] = fast_exp2(s[1][h] - mu);
      l[h] += p[0][h] + p[1][h];
    }

    // P.V
    if constexpr (BF16) {
      uint32_t pp[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pp[h] = pack_bf16x2(p[0][h], p[1][h]);
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = u4(vr[x][0][hh], w), a1 = u4(vr[x][1][hh], w);
          const uint32_t plo = pair_lo(a0, a1), phi = pair_hi(a0, a1);
          const int e = hh * VEC + 2 * w;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            o[h][e] = dot2_bf16(pp[h], plo, o[h][e]);
            o[h][e + 1] = dot2_bf16(pp[h], phi, o[h][e + 1]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          float vf[VEC];
          widen<BF16, VEC>(vr[x][u][hh], vf);
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              o[h][hh * VEC + e] = fmaf(p[u][h], vf[e], o[h][hh * VEC + e]);
        }
      }
    }
    }
  }

  // merge the 8 token rows of the wave (lanes c, c+8, ...)
#pragma unroll
  for (int d = 8; d < 64; d <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], d);
      const float lo = __shfl_xor(l[h], d);
      const float mn = fmaxf(m[h], mo);
      const float mu = mn == NEG_INF ? 0.f : mn;
      const float a1 = fast_exp2(m[h] - mu), a2 = fast_exp2(mo - mu);
      l[h] = l[h] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[h][e] = o[h][e] * a1 + __shfl_xor(o[h][e], d) * a2;
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
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm_o[wave][h][hh * SEG + c * VEC + e] = o[h][hh * VEC + e];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  const size_t row0 = (size_t)b * a.Hq + (size_t)kvh * G;
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
    const size_t row = row0 + h;
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

template <bool BF16, int D, bool FAST>
hipError_t launch_df(const GqaArgs& a, hipStream_t s) {
  dim3 grid(a.num_splits, a.Hkv, a.B), block(kThreads);
  switch (a.G) {
    case 1: gqa_split_kernel<BF16, D, 1, FAST><<<grid, block, 0, s>>>(a); break;
    case 2: gqa_split_kernel<BF16, D, 2, FAST><<<grid, block, 0, s>>>(a); break;
    case 4: gqa_split_kernel<BF16, D, 4, FAST><<<grid, block, 0, s>>>(a); break;
    case 8: gqa_split_kernel<BF16, D, 8, FAST><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_d(const GqaArgs& a, hipStream_t s) {
  const bool fast = !a.page_table || a.page_size % kStep == 0;
  return fast ? launch_df<BF16, D, true>(a, s) : launch_df<BF16, D, false>(a, s);
}

template <bool BF16, int D, bool FAST>
int occupancy_g(int G) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (G) {
    case 1: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_split_kernel<BF16, D, 1, FAST>, kThreads, 0); break;
    case 2: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_split_kernel<BF16, D, 2, FAST>, kThreads, 0); break;
    case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_split_kernel<BF16, D, 4, FAST>, kThreads, 0); break;
    case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gqa_split_kernel<BF16, D, 8, FAST>, kThreads, 0); break;
  }
  return e == hipSuccess ? n : 0;
}

// Merge split partials (o_j normalised, lse_j in log2 units):
// lse = max + log2 sum_j 2^(lse_j - max); o = sum_j 2^(lse_j - lse) o_j.
// One thread per output element; it loads its row's split log-sum-exps and
// its split partials together (one memory round trip), then merges.  Splits
// may also hand over unnormalised sums with their reference maximum and
// softmax denominator (CombineArgs::part_l): the same merge with weights
// 2^(m - M) on both the sums and the denominators.
constexpr int kCombineThreads = 256;
constexpr int kMaxCombineSplits = 256;
constexpr int kCombineChunk = 16;

template <bool BF16>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(const CombineArgs a) {
  const float NEG_INF = -__builtin_inff();
  const size_t e = (size_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (e >= (size_t)a.rows * a.D) return;
  const int row = (int)(e / a.D), d = (int)(e % a.D);
  const int S = a.splits;
  const float* pl = a.part_lse + (size_t)row * S;
  const float* ps = a.part_l ? a.part_l + (size_t)row * S : nullptr;
  const float* po = a.part_o + (size_t)row * S * a.D + d;
  float M = NEG_INF, wsum = 0.f, acc = 0.f;
  for (int j0 = 0; j0 < S; j0 += kCombineChunk) {
    float x[kCombineChunk], v[kCombineChunk], l[kCombineChunk];
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const bool in = j0 + u < S;
      x[u] = in ? pl[j0 + u] : NEG_INF;
      v[u] = in ? po[(size_t)(j0 + u) * a.D] : 0.f;
      l[u] = ps && in ? ps[j0 + u] : 1.f;
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) Mc = fmaxf(Mc, x[u]);
    const float mu = Mc == NEG_INF ? 0.f : Mc;
    const float f = fast_exp2(M - mu);  // rescales the running sums (0 while M is -inf)
    wsum *= f;
    acc *= f;
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const float w = fast_exp2(x[u] - mu);
      wsum = fmaf(w, l[u], wsum);
      acc = fmaf(w, v[u], acc);
    }
    M = Mc;
  }
  const float val = wsum > 0.f ? acc / wsum : 0.f;
  if constexpr (BF16) ((uint16_t*)a.out)[e] = f32_to_bf16(val);
  else ((float*)a.out)[e] = val;
  if (d == 0 && a.lse) a.lse[row] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : NEG_INF;
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

int gqa_blocks_per_cu(bool bf16, int D, int G, bool paged, int page_size) {
  const bool fast = !paged || page_size % kStep == 0;
  if (bf16) {
    if (D == 64) return fast ? occupancy_g<true, 64, true>(G) : occupancy_g<true, 64, false>(G);
    return fast ? occupancy_g<true, 128, true>(G) : occupancy_g<true, 128, false>(G);
  }
  if (D == 64) return fast ? occupancy_g<false, 64, true>(G) : occupancy_g<false, 64, false>(G);
  return fast ? occupancy_g<false, 128, true>(G) : occupancy_g<false, 128, false>(G);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.splits > kMaxCombineSplits) return hipErrorInvalidValue;
  const size_t total = (size_t)a.rows * a.D;
  const unsigned blocks = (unsigned)((total + kCombineThreads - 1) / kCombineThreads);
  if (a.bf16) lse_combine_kernel<true><<<blocks, kCombineThreads, 0, s>>>(a);
  else lse_combine_kernel<false><<<blocks, kCombineThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dattn
