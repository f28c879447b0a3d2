// Absorbed MLA decode attention over a 576-wide latent cache, dense or over a
// gathered top-k token list (sparse MLA), on bf16 MFMA.
//
// Every query head reads the same latent row [c_KV (512) | k_pe (64)]
// ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
// Path"; with W_UK absorbed into the query, "Overview of Attention
// Mechanism", MLA), so the scores of a tile of tokens for many heads are one
// dense product, and so is P.c_KV.  A workgroup owns (sequence, 64 heads,
// token split); each of its 4 waves owns 16 heads.
//
// Per 32-token tile:
//   * the tile's 32 x 1152 B of latent rows is staged in LDS, row-major, with
//     the 16-byte chunks of row r permuted by c ^ f(r) so that both read
//     patterns below are free of bank conflicts;
//   * S^T[token, head] = C[token, :] . Q^T over 576 dims: 16x16x32 bf16 MFMA,
//     A = latent chunks from LDS, B = the wave's query (registers, loaded once);
//   * online softmax in log2 units per head (running max and sum, earlier
//     partials rescaled -- "All the attentions", section 1);
//   * O[head, 0:512] += P . C[:, 0:512]: the accumulator layout of S^T is
//     exactly the A operand layout P needs (heads x tokens), and the B operand
//     (tokens x dims) is read from the row-major tile by the gfx950 transpose
//     read ds_read_b64_tr_b16, so V is never copied or transposed.
// P is rounded to bf16 for the MFMA; everything else accumulates in fp32.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kDc = 512;            // c_KV width (the value)
constexpr int kDq = 576;            // latent row: c_KV + k_pe
constexpr int kChunks = kDq / 8;    // 16-byte chunks per row
constexpr int kTile = 32;           // tokens per tile
constexpr int kWaves = 4;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerWG = kWaves * kHeadsPerWave;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileChunks = kTile * kChunks;            // 2304
constexpr int kLoadsPerThread = kTileChunks / kThreads; // 9
static_assert(kTileChunks % kThreads == 0, "tile split");
constexpr int kTileBytes = kTileChunks * 16;            // 36864
constexpr int kQBytes = kHeadsPerWG * kDq * 2;          // 73728
constexpr int kQChunks = kHeadsPerWG * kChunks;         // 4608
static_assert(kQChunks % kThreads == 0, "q split");
constexpr int kLdsBytes = kTileBytes + kQBytes;

// chunk permutation of row r (low three bits of the chunk index only)
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int chunk_off(int r, int c) { return r * (kDq * 2) + 16 * (c ^ swz(r)); }

template <bool SPARSE, bool PAGED>
__global__ __launch_bounds__(kThreads, 1) void mla_split_kernel(const MlaArgs a) {
  const float NEG_INF = -__builtin_inff();
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* tile = lds;
  char* qlds = lds + kTileBytes;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;     // 16-lane group
  const int li = lane & 15;
  const int split = blockIdx.x;
  const int h0 = blockIdx.y * kHeadsPerWG + wave * kHeadsPerWave;
  const int b = blockIdx.z;

  const int N = SPARSE ? a.k_sel : a.seq_lens[b];
  const int per = ((N + a.num_splits - 1) / a.num_splits + kTile - 1) / kTile * kTile;
  const int f_begin = split * per;
  const int f_end = min(N, f_begin + per);
  const int n_tiles = f_end > f_begin ? (f_end - f_begin + kTile - 1) / kTile : 0;

  // the workgroup's 64 query rows, staged once in LDS with the tile's chunk
  // permutation (rows = heads); B operand of S^T = C Q^T
  {
    const uint16_t* qsrc = a.q + ((size_t)b * a.H + blockIdx.y * kHeadsPerWG) * kDq;
    for (int P = threadIdx.x; P < kQChunks; P += kThreads) {
      const int r = P / kChunks, c = P % kChunks;
      *(uint4*)(qlds + chunk_off(r, c)) = *(const uint4*)(qsrc + (size_t)r * kDq + 8 * c);
    }
  }
  const int qrow = wave * kHeadsPerWave + li;

  // global source of the tile chunks this thread stages
  auto row_ptr = [&](int f) -> const uint16_t* {
    if (f >= f_end) return nullptr;
    int t;
    if constexpr (SPARSE) {
      t = a.idx[(size_t)b * a.k_sel + f];
      if (t < 0) return nullptr;
    } else {
      t = f;
    }
    size_t row;
    if constexpr (PAGED) {
      const int phys = a.page_table[(size_t)b * a.max_pages + (t >> a.log2_page)];
      row = (size_t)phys * a.page_size + (t & (a.page_size - 1));
    } else {
      row = (size_t)b * a.S_max + t;
    }
    return a.latent + row * kDq;
  };

  uint4 stage[kLoadsPerThread];
  auto load_tile = [&](int tix) {
    const int base = f_begin + tix * kTile;
#pragma unroll
    for (int k = 0; k < kLoadsPerThread; ++k) {
      const int P = threadIdx.x + kThreads * k;
      const int r = P / kChunks, c = P % kChunks;
      const uint16_t* src = row_ptr(base + r);
      stage[k] = src ? *(const uint4*)(src + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < kLoadsPerThread; ++k) {
      const int P = threadIdx.x + kThreads * k;
      const int r = P / kChunks, c = P % kChunks;
      *(uint4*)(tile + chunk_off(r, c)) = stage[k];
    }
  };

  f32x4_t acc[kDc / 16];
#pragma unroll
  for (int n = 0; n < kDc / 16; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;

  if (n_tiles > 0) load_tile(0);
  for (int tix = 0; tix < n_tiles; ++tix) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tix + 1 < n_tiles) load_tile(tix + 1);
    const int base = f_begin + tix * kTile;

    // S^T for tokens [16m, 16m+16) of the tile: lane holds tokens 16m+4g+v, head li
    f32x4_t st[2];
    st[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      // one k-step of A fragments in flight ahead of the MFMAs
      uint4 a0 = *(const uint4*)(tile + chunk_off(li, g));
      uint4 a1 = *(const uint4*)(tile + chunk_off(16 + li, g));
      uint4 q0 = *(const uint4*)(qlds + chunk_off(qrow, g));
#pragma unroll
      for (int ks = 0; ks < kDq / 32; ++ks) {
        uint4 n0 = a0, n1 = a1, nq = q0;
        if (ks + 1 < kDq / 32) {
          n0 = *(const uint4*)(tile + chunk_off(li, 4 * (ks + 1) + g));
          n1 = *(const uint4*)(tile + chunk_off(16 + li, 4 * (ks + 1) + g));
          nq = *(const uint4*)(qlds + chunk_off(qrow, 4 * (ks + 1) + g));
        }
        st[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                        __builtin_bit_cast(bf16x8_t, q0),
                                                        st[0], 0, 0, 0);
        st[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                        __builtin_bit_cast(bf16x8_t, q0),
                                                        st[1], 0, 0, 0);
        a0 = n0;
        a1 = n1;
        q0 = nq;
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // online softmax (log2 units); tokens past the split end or empty top-k slots score -inf
    float s[2][4];
    float mx = NEG_INF;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int f = base + 16 * mt + 4 * g + v;
        bool ok = f < f_end;
        if constexpr (SPARSE) ok = ok && a.idx[(size_t)b * a.k_sel + f] >= 0;
        const float x = ok ? st[mt][v] * a.scale_log2 : NEG_INF;
        s[mt][v] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float mu = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mu);
    m_run = m_new;
    float p[2][4], psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[mt][v] = fast_exp2(s[mt][v] - mu);
        psum += p[mt][v];
      }
    }
    l_run = l_run * alpha + psum;

    // A operand of P.V: head li, tokens (4g..4g+3, 16+4g..16+4g+3)
    uint4 pa;
    pa.x = pack_bf16x2(p[0][0], p[0][1]);
    pa.y = pack_bf16x2(p[0][2], p[0][3]);
    pa.z = pack_bf16x2(p[1][0], p[1][1]);
    pa.w = pack_bf16x2(p[1][2], p[1][3]);

    // rescale O rows (heads 4g+v) by their heads' alpha
    if (__any(alpha != 1.f)) {
      float av[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * g + v);
#pragma unroll
      for (int n = 0; n < kDc / 16; ++n) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[n][v] *= av[v];
      }
    }

    // O += P . V, V read transposed from the row-major tile
    const int rr1 = 4 * g + (li >> 2);       // tokens of k elements 0..3
    const int rr2 = 16 + 4 * g + (li >> 2);  // tokens of k elements 4..7
    const int dsub = 4 * (li & 3);
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    typedef __attribute__((address_space(3))) char lds_char;
    auto vread = [&](int n) -> bf16x8_t {
      const int d = 16 * n + dsub;
      const int c = d >> 3, bo = (d & 7) * 2;
      const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)((lds_char*)tile + chunk_off(rr1, c) + bo));
      const bf16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4*)((lds_char*)tile + chunk_off(rr2, c) + bo));
      return __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    const bf16x8_t pab = __builtin_bit_cast(bf16x8_t, pa);
    bf16x8_t vb = vread(0);
#pragma unroll
    for (int n = 0; n < kDc / 16; ++n) {
      bf16x8_t vn = vb;
      if (n + 1 < kDc / 16) vn = vread(n + 1);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pab, vb, acc[n], 0, 0, 0);
      vb = vn;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // totals per head: sum partial l over the 4 lane groups
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : NEG_INF;
  float inv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float lv = __shfl(l_tot, 4 * g + v);
    inv[v] = lv > 0.f ? 1.f / lv : 0.f;
  }
  const size_t row0 = (size_t)b * a.H + h0;
  if (a.num_splits == 1) {
#pragma unroll
    for (int n = 0; n < kDc / 16; ++n) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        a.out[(row0 + 4 * g + v) * kDc + 16 * n + li] = f32_to_bf16(acc[n][v] * inv[v]);
    }
    if (g == 0 && a.lse) a.lse[row0 + li] = lse2 == NEG_INF ? NEG_INF : lse2 * kLn2;
  } else {
#pragma unroll
    for (int n = 0; n < kDc / 16; ++n) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        a.part_o[((row0 + 4 * g + v) * a.num_splits + split) * kDc + 16 * n + li] = acc[n][v] * inv[v];
    }
    if (g == 0) a.part_lse[(row0 + li) * a.num_splits + split] = lse2;
  }
}

template <bool SPARSE, bool PAGED>
hipError_t launch_variant(const MlaArgs& a, hipStream_t s) {
  static bool configured = false;  // the attribute is per function, set once
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)mla_split_kernel<SPARSE, PAGED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  dim3 grid(a.num_splits, a.H / kHeadsPerWG, a.B), block(kThreads);
  mla_split_kernel<SPARSE, PAGED><<<grid, block, kLdsBytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaArgs& a, hipStream_t s) {
  if (a.idx) return launch_variant<true, false>(a, s);
  if (a.page_table) return launch_variant<false, true>(a, s);
  return launch_variant<false, false>(a, s);
}

}  // namespace dattn
