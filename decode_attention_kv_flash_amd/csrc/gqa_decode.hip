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
// one wave-uniform scalar table lookup, and a lane's addresses are fixed
// offsets from it.  The set's partial first and last blocks are masked per
// token.  Inside a workgroup each wave streams its own blocks:
//   * a lane holds one 16-byte piece of a token row: LPR = row bytes / 16
//     lanes cover a row, one wave load instruction reads 64 / LPR whole rows,
//     and a lane holds 16 * LPR / 64 rows of a block for K and as many for V;
//   * one register buffer per wave, loaded and then consumed; latency is
//     hidden across waves (a small register footprint keeps several
//     workgroups resident per CU, so one wave's loads overlap another's
//     arithmetic), and the page of the wave's next block is looked up one
//     step ahead.  Eight bf16 heads per KV head fill the register file, two
//     waves per SIMD: those kernels keep two buffers per wave and issue the
//     next block's loads before this block's arithmetic;
//   * scores are lane-partial dot products (v_dot2_f32_bf16 for bf16: the
//     bf16 products are exact in fp32) summed over the row's lanes with DPP;
//   * the softmax is the online one ("All the attentions", section 1: a
//     running maximum and running sum, earlier partials rescaled), kept per
//     token row of lanes; the reference maximum only moves when the new
//     maximum exceeds it by more than 2^8, which bounds every exponential by
//     2^8 and makes rescaling rare without changing the result;
//   * with 16 lanes per token row (D = 128 bf16 or D = 64 fp32) or 8 (D = 64
//     bf16) and four or eight heads per KV head, the sum over the row is a
//     transposing one that leaves each lane one score per block of four
//     heads; the lane takes that score's exponential and the probabilities
//     are broadcast back with DPP (one exponential per lane and block instead
//     of one per score of the block);
//   * P.V: for bf16 the probabilities of two tokens are rounded to bf16 and
//     paired with the two tokens' values in one v_dot2_f32_bf16 per output
//     (fp32 accumulation); for fp32 inputs it is plain fp32 FMA.
// A split's result is (o / l, log2-sum-exp); lse_combine merges the splits
// (lse = max + log2 sum 2^(lse_j - max), o = sum 2^(lse_j - lse) o_j).
//
// The same kernel attends a listed token set (query-aware page selection,
// "Long context, KV eviction and sparse attention", "Sparse attention:
// choosing dynamically at every step"): per query head a list of 16-token
// blocks plus the partial last block, either one query head per workgroup
// or, for a group of heads sharing a KV head, the union of their lists with
// the heads that chose each block, so that a block two heads chose is read
// once.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 16;     // tokens per wave step (one block)
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

template <bool BF16, int D>
struct GqaShape {
  static constexpr int ESZ = BF16 ? 2 : 4;   // bytes per element
  static constexpr int VEC = 16 / ESZ;       // elements of a row one lane holds
  static constexpr int LPR = D / VEC;        // lanes per token row
  static constexpr int RPI = 64 / LPR;       // token rows per wave load
  static constexpr int TPL = kStep / RPI;    // token rows per lane per block
  static_assert(D % VEC == 0 && LPR >= 8 && LPR <= 32 && TPL % 2 == 0, "row split");
};

// One block of K and V held by a lane: TPL token rows, one 16-byte piece each.
template <int TPL>
struct KvRegs {
  uint4 k[TPL], v[TPL];
};

typedef const int32_t __attribute__((address_space(4))) cint32_t;

__device__ __forceinline__ uint32_t u4(const uint4& x, int w) {
  return w == 0 ? x.x : w == 1 ? x.y : w == 2 ? x.z : x.w;
}

template <int N>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (N == 8 || N == 16) {
    return group_sum<N>(x);
  } else {
    static_assert(N == 32, "lanes per row");
    x = group_sum<16>(x);
    return x + __shfl_xor(x, 16);
  }
}

// Broadcast of lane N of each 16-lane row to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ uint32_t row_bcast_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + N, 0xF, 0xF, false);
}

// row_bcast_u32 by a lane index known after unrolling.
__device__ __forceinline__ uint32_t row_bcast_at(uint32_t x, int n) {
  switch (n) {
    case 0: return row_bcast_u32<0>(x);
    case 1: return row_bcast_u32<1>(x);
    case 2: return row_bcast_u32<2>(x);
    case 3: return row_bcast_u32<3>(x);
    case 4: return row_bcast_u32<4>(x);
    case 5: return row_bcast_u32<5>(x);
    case 6: return row_bcast_u32<6>(x);
    case 7: return row_bcast_u32<7>(x);
    case 8: return row_bcast_u32<8>(x);
    case 9: return row_bcast_u32<9>(x);
    case 10: return row_bcast_u32<10>(x);
    case 11: return row_bcast_u32<11>(x);
    case 12: return row_bcast_u32<12>(x);
    case 13: return row_bcast_u32<13>(x);
    case 14: return row_bcast_u32<14>(x);
    default: return row_bcast_u32<15>(x);
  }
}
__device__ __forceinline__ float row_bcast_at(float x, int n) {
  return __uint_as_float(row_bcast_at(__float_as_uint(x), n));
}

// Broadcast of lane N of each 8-lane group to the group: a quad broadcast
// (quad_perm [N, N, N, N] mod 4), after which the group's other quad takes
// the value from four lanes away (a row shift written to that quad's DPP
// banks only; bank k is lanes 4k .. 4k + 3 of a 16-lane row).
template <int N>
__device__ __forceinline__ uint32_t half_bcast_u32(uint32_t x) {
  const int y = __builtin_amdgcn_update_dpp(0, (int)x, (N & 3) * 0x55, 0xF, 0xF, false);
  if constexpr (N < 4)  // lanes 4..7 of the group read lane j - 4 (row_shr:4)
    return (uint32_t)__builtin_amdgcn_update_dpp(y, y, 0x114, 0xF, 0xA, false);
  else  // lanes 0..3 read lane j + 4 (row_shl:4)
    return (uint32_t)__builtin_amdgcn_update_dpp(y, y, 0x104, 0xF, 0x5, false);
}

__device__ __forceinline__ uint32_t half_bcast_at(uint32_t x, int n) {
  switch (n) {
    case 0: return half_bcast_u32<0>(x);
    case 1: return half_bcast_u32<1>(x);
    case 2: return half_bcast_u32<2>(x);
    case 3: return half_bcast_u32<3>(x);
    case 4: return half_bcast_u32<4>(x);
    case 5: return half_bcast_u32<5>(x);
    case 6: return half_bcast_u32<6>(x);
    default: return half_bcast_u32<7>(x);
  }
}

// Lane n of each LPR-lane group (a token row) to the whole group.
template <int LPR>
__device__ __forceinline__ uint32_t group_bcast_at(uint32_t x, int n) {
  static_assert(LPR == 8 || LPR == 16, "group of 8 or 16 lanes");
  if constexpr (LPR == 16) return row_bcast_at(x, n);
  else return half_bcast_at(x, n);
}
template <int LPR>
__device__ __forceinline__ float group_bcast_at(float x, int n) {
  return __uint_as_float(group_bcast_at<LPR>(__float_as_uint(x), n));
}

// Transposing sum over the NV = 16 (or 8) lanes of a row of values
// numbered TPL i + u (head i < 4 of a block, token row u < TPL = NV / 4).
// Each step pairs a lane with a partner (15 - c by row_mirror, c ^ 7 within
// the 8-lane half by row_half_mirror, then the quad swaps c ^ 2 and c ^ 1;
// with eight lanes the first step is left out) and halves the values the
// lane holds, so that it ends with the row's total of one of them: NV - 1
// adds instead of the NV log2(NV) of summing every value in every lane.
//   * The first two steps split the heads.  Lane c keeps its values in the
//     order v[TPL i + u] = (its part of head i ^ gray(c / TPL), token row u),
//     fixed per lane by the order it loads its query rows in (gray(q) = q ^
//     (q >> 1)); with that order the partners' upper halves always hold the
//     lane's lower half's heads, and the lane just adds them.
//   * The last steps split the token rows between the TPL lanes of a head:
//     there the lane keeps the half its own bit selects and adds the
//     partner's copy of that half.
// Lane c ends with head gray(c / TPL), token row c % TPL; xpose_lane(i, u)
// is the lane that ends with head i, token row u.
__host__ __device__ constexpr int gray2(int q) { return q ^ (q >> 1); }
template <int TPL>
__host__ __device__ constexpr int xpose_lane(int i, int u) {
  return TPL * gray2(i) + u;  // gray2 is its own inverse on two bits
}

template <int CTRL, int N, int NV>
__device__ __forceinline__ void xpose_add(float (&v)[NV]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<CTRL>(v[i + N]);
}

template <int CTRL, int N, int NV>
__device__ __forceinline__ void xpose_keep(float (&v)[NV], bool upper) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = upper ? v[i + N] : v[i];
    const float send = upper ? v[i] : v[i + N];
    v[i] = keep + dpp_f32<CTRL>(send);
  }
}

template <int NV>
__device__ __forceinline__ float xpose_sum(float (&v)[NV], int c) {
  static_assert(NV == 8 || NV == 16, "eight or sixteen lanes");
  if constexpr (NV == 16) {
    xpose_add<0x140, 8>(v);      // partner 15 - c: heads
    xpose_add<0x141, 4>(v);      // partner c ^ 7 within the half: heads
    xpose_keep<0x4E, 2>(v, c & 2);  // partner c ^ 2: token rows
  } else {
    xpose_add<0x141, 4>(v);      // partner c ^ 7: heads
    xpose_add<0x4E, 2>(v);       // partner c ^ 2: heads
  }
  xpose_keep<0xB1, 1>(v, c & 1);  // partner c ^ 1: token rows
  return v[0];
}

// PAGED_FAST: paged with page_size % 16 == 0, or contiguous (one lookup per
// block); otherwise every token resolves its own page.
// SET: which tokens a query head attends.
//   kSetWindow: [0, L) or window + sinks;
//   kSetPerHead: a list of 16-token blocks per query head (the pages a
//     query-aware selection chose, ascending, -1 padded) plus the partial
//     last block; one query head per workgroup (G = 1), reading KV head
//     h / (Hq / Hkv);
//   kSetUnion: the union of the G heads' block lists, ascending, each entry
//     block | heads << 24 (the heads that chose it), plus the partial last
//     block: every chosen block is read once for the whole group and
//     attended by the heads that chose it only.
constexpr int kSetWindow = 0, kSetPerHead = 1, kSetUnion = 2;

// (At least three waves per SIMD: only the eight-head instances are near
// the limit, and three of them with a register or two spilled beat two.)
// Eight bf16 heads per KV head keep two register buffers per wave (see the
// main loop) and run two waves per SIMD.
template <bool BF16, int G>
constexpr bool gqa_double_buffer() { return BF16 && G >= 8; }

template <bool BF16, int D, int G, bool PAGED_FAST, int SET = kSetWindow>
__global__ __launch_bounds__(kThreads, (gqa_double_buffer<BF16, G>() ? 2 : 3)) void gqa_split_kernel(
    const GqaArgs a) {
  using S = GqaShape<BF16, D>;
  constexpr int VEC = S::VEC, LPR = S::LPR, RPI = S::RPI, TPL = S::TPL;
  const float NEG_INF = -__builtin_inff();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;  // token row within one wave load
  const int c = lane % LPR;  // 16-byte piece of the row
  const int split = blockIdx.x;
  constexpr bool LISTED = SET != kSetWindow;
  static_assert(SET != kSetPerHead || G == 1, "a per-head token set has one head per workgroup");
  const int qh0 = SET == kSetPerHead ? (int)blockIdx.y : (int)blockIdx.y * G;  // first query head
  const int kvh = SET == kSetPerHead ? (int)blockIdx.y / a.G : (int)blockIdx.y;
  const int b = blockIdx.z;

  // Token set [0, s_cnt) u [w_start, L) as 16-token blocks: sink blocks
  // first, then the window's blocks (aligned down to 16).  LISTED: the
  // listed blocks, then the partial last block.
  // seq_lens is a caller contract; clamping keeps an out-of-contract length
  // inside the sequence's row of the page table (and the cache)
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), (int64_t)a.page_size * a.max_pages);
  int s_cnt = 0, w_start = 0;
  if (!LISTED && a.window > 0 && a.window < L) {
    w_start = L - a.window;
    s_cnt = min(a.n_sink, w_start);
  }
  const int n_full = L / kStep;
  const int n_listed = SET == kSetUnion ? a.list_count[b * a.Hkv + kvh] : a.list_len;
  const int n_sb = LISTED ? min(n_listed, n_full) : (s_cnt + kStep - 1) / kStep;
  const int wb0 = w_start / kStep;
  const int n_wb = LISTED ? (L % kStep != 0) : L > 0 ? (L + kStep - 1) / kStep - wb0 : 0;
  const int n_blocks = n_sb + n_wb;
  const size_t list_row = SET == kSetUnion ? (size_t)b * a.Hkv + kvh : (size_t)b * a.Hq + qh0;
  const cint32_t* list = LISTED ? (const cint32_t*)(uintptr_t)(a.block_list + list_row * a.list_len) : nullptr;
  const int per = (n_blocks + a.num_splits - 1) / a.num_splits;
  const int blk_begin = min(n_blocks, split * per);
  const int blk_end = min(n_blocks, blk_begin + per);

  // With LPR = 16 (or 8) lanes per token row and as many (token row, head)
  // scores per lane and block of four heads (four heads times TPL = LPR / 4
  // token rows) the softmax runs transposed: after the transposing sum,
  // lane c of the row owns one score of each block of four heads: head
  // xi = gray(c / TPL) of the block, token row xu = c % TPL of the step.  It
  // takes one exponential (not LPR copies of each), and the probabilities
  // are broadcast back for P.V.  For the sum, the lane's query slot i holds
  // head i ^ xi of each block.
  constexpr bool kXpose = (LPR == 16 || LPR == 8) && LPR == 4 * TPL && (G == 4 || G == 8);
  constexpr int kNB = G >= 4 ? G / 4 : 1;  // blocks of LPR (token row, head) scores per lane
  const int xu = kXpose ? c % TPL : 0, xi = kXpose ? gray2(c / TPL) : 0;

  // This lane's piece of each of the G query rows: dims c*VEC + [0, VEC).
  uint4 qv[G];
  {
    const char* qb = (const char*)a.q + ((size_t)(b * a.Hq + qh0) * D + c * VEC) * S::ESZ;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int hs = kXpose ? (h & ~3) | ((h & 3) ^ xi) : h;
      qv[h] = *(const uint4*)(qb + (size_t)hs * D * S::ESZ);
    }
  }

  float m[G], l[G], o[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = NEG_INF;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
  }
  // Transposed softmax: lc is the lane's share of its head's denominator,
  // mo the reference maximum of its head (m of that head).
  float lc[kNB], mo[kNB];
#pragma unroll
  for (int k = 0; k < kNB; ++k) {
    lc[k] = 0.f;
    mo[k] = NEG_INF;
  }

  const size_t head_stride = (size_t)a.page_size * D;
  const size_t page_stride = (size_t)a.Hkv * head_stride;
  const char* kb = (const char*)a.k;
  const char* vb = (const char*)a.v;
  // The page table is read-only for the whole launch: reading it through the
  // constant address space lets wave-uniform lookups become scalar loads.
  const cint32_t* pt = a.page_table ? (const cint32_t*)(uintptr_t)(a.page_table + (size_t)b * a.max_pages)
                                    : nullptr;
  const size_t contig_base = ((size_t)b * a.Hkv + kvh) * head_stride;
  const size_t lane_off = (size_t)c * 16;

  auto block_start = [&](int blk) {
    if constexpr (SET == kSetUnion) return (blk < n_sb ? (int)((uint32_t)list[blk] & 0xffffffu) : n_full) * kStep;
    if constexpr (SET == kSetPerHead) return (blk < n_sb ? max((int)list[blk], 0) : n_full) * kStep;
    return blk < n_sb ? blk * kStep : (wb0 + blk - n_sb) * kStep;
  };
  // Attended token range [lo, hi) inside block blk (never empty for a block
  // below blk_end).
  auto block_range = [&](int blk, int t0, int& lo, int& hi) {
    if constexpr (LISTED) {
      lo = t0;
      hi = min(L, t0 + kStep);
      return;
    }
    const bool sink = blk < n_sb;
    lo = max(sink ? 0 : w_start, t0);
    hi = min(sink ? s_cnt : L, t0 + kStep);
  };
  // Physical page of a block (wave-uniform; PAGED_FAST with a page table).
  auto page_of = [&](int blk) { return (int)pt[block_start(blk) >> a.log2_page]; };

  // Byte offsets of the lane's rows inside a 16-token block (the rows of a
  // block are contiguous in the page).
  uint32_t roff[TPL];
#pragma unroll
  for (int u = 0; u < TPL; ++u) roff[u] = (uint32_t)(((u * RPI + r) * D) * S::ESZ) + (uint32_t)lane_off;

  // Issue the K/V loads of block blk (< blk_end) into R.  In a partial block
  // a lane whose token is outside the attended range loads the nearest
  // attended row of the block instead: every address stays inside a page the
  // table names (or inside the contiguous sequence), nothing past L_b is
  // read, and the row is masked at compute time, so the loads need no
  // branches.  A whole block takes the lane's fixed row offsets from one
  // wave-uniform base.
  auto issue = [&](int blk, int phys, KvRegs<TPL>& R) {
    const int t0 = block_start(blk);
    int lo, hi;
    block_range(blk, t0, lo, hi);
    if constexpr (PAGED_FAST) {
      const size_t base = (pt ? (size_t)phys * page_stride + (size_t)kvh * head_stride +
                                    (size_t)(t0 & (a.page_size - 1)) * D
                              : contig_base + (size_t)t0 * D) * S::ESZ;
      const char* kp = kb + base;
      const char* vp = vb + base;
      const bool whole = lo == t0 && hi == t0 + kStep;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        // one load sequence for whole and partial blocks (the waits before
        // the arithmetic then count loads exactly), each load the scalar
        // base plus the lane's 32-bit offset
        const uint32_t ro = whole ? roff[u]
                                  : (uint32_t)((min(max(t0 + u * RPI + r, lo), hi - 1) - t0) * D * S::ESZ) +
                                        (uint32_t)lane_off;
        R.k[u] = load_stream(kp + ro);
        R.v[u] = load_stream(vp + ro);
      }
    } else {
      auto off_of = [&](int t) {
        const int ph = a.page_table[(size_t)b * a.max_pages + (t >> a.log2_page)];
        return ((size_t)ph * page_stride + (size_t)kvh * head_stride + (size_t)(t & (a.page_size - 1)) * D) *
                   S::ESZ + lane_off;
      };
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const size_t off = off_of(min(max(t0 + u * RPI + r, lo), hi - 1));
        R.k[u] = load_stream(kb + off);
        R.v[u] = load_stream(vb + off);
      }
    }
  };

  // The transposed path of compute (kXpose): tokens t0 + u RPI + r, u < TPL;
  // block k of the scores holds heads 4k .. 4k + 3.
  auto compute_xpose = [&](int t0, int lo, int hi, uint32_t heads, const KvRegs<TPL>& R) {
    if constexpr (kXpose) {
      float dot[kNB];
      // one block of four heads at a time: its LPR partial dot products are
      // transposed before the next block's are formed (fewer live registers)
#pragma unroll
      for (int k = 0; k < kNB; ++k) {
        float v[LPR];  // v[TPL i + u]: this lane's part of q_{4k + (i ^ xi)} . k_u
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = 4 * k + i;
            float acc;
            if constexpr (BF16) {
              acc = dot2_bf16_first(R.k[u].x, qv[h].x);
              acc = dot2_bf16(R.k[u].y, qv[h].y, acc);
              acc = dot2_bf16(R.k[u].z, qv[h].z, acc);
              acc = dot2_bf16(R.k[u].w, qv[h].w, acc);
            } else {
              acc = __uint_as_float(R.k[u].x) * __uint_as_float(qv[h].x);
              acc = fmaf(__uint_as_float(R.k[u].y), __uint_as_float(qv[h].y), acc);
              acc = fmaf(__uint_as_float(R.k[u].z), __uint_as_float(qv[h].z), acc);
              acc = fmaf(__uint_as_float(R.k[u].w), __uint_as_float(qv[h].w), acc);
            }
            v[TPL * i + u] = acc;
          }
        }
        // every lane of the row takes part in the cross-lane sum (a lane
        // left out would hand its partners zeros): sum first, then mask
        dot[k] = xpose_sum<LPR>(v, c);
      }
      const int t = t0 + xu * RPI + r;
      const bool tvalid = t >= lo && t < hi;
      float sc[kNB];
      bool up = false;
#pragma unroll
      for (int k = 0; k < kNB; ++k) {
        sc[k] = tvalid && ((heads >> (4 * k + xi)) & 1u) ? dot[k] * a.scale_log2 : NEG_INF;
        up = up || sc[k] > mo[k] + kTau;
      }
      // The reference maxima move only when a score passes its head's by
      // more than kTau, which is rare after the first block: the wave takes
      // the branch only then.  In it each head's maximum over the row's TPL
      // tokens goes to every lane of the row (the maxima are kept per row,
      // in every lane).
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
        float mxh[G];
#pragma unroll
        for (int k = 0; k < kNB; ++k) {
          float mx = fmaxf(sc[k], dpp_f32<0xB1>(sc[k]));
          if constexpr (TPL == 4) mx = fmaxf(mx, dpp_f32<0x4E>(mx));
#pragma unroll
          for (int i = 0; i < 4; ++i) mxh[4 * k + i] = group_bcast_at<LPR>(mx, xpose_lane<TPL>(i, 0));
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const bool own = xi == (h & 3);  // this lane holds head h in block h / 4
          if (mxh[h] > m[h] + kTau) {
            const float alpha = fast_exp2(m[h] - mxh[h]);  // 0 when m was -inf
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[h][e] *= alpha;
            if (own) lc[h / 4] *= alpha;
            m[h] = mxh[h];
          }
          if (own) mo[h / 4] = m[h];
        }
      }
      float p[kNB];
#pragma unroll
      for (int k = 0; k < kNB; ++k) {
        p[k] = fast_exp2(sc[k] - (mo[k] == NEG_INF ? 0.f : mo[k]));
        lc[k] += p[k];
      }
      if constexpr (BF16) {
        // (p_u, p_u+1) of a head in the lanes of even u, then to every lane
        uint32_t pk[kNB];
#pragma unroll
        for (int k = 0; k < kNB; ++k) pk[k] = pack_bf16x2(p[k], dpp_f32<0xB1>(p[k]));
#pragma unroll
        for (int j = 0; j < TPL / 2; ++j) {
          uint32_t pp[G];
#pragma unroll
          for (int h = 0; h < G; ++h)
            pp[h] = group_bcast_at<LPR>(pk[h / 4], xpose_lane<TPL>(h % 4, 2 * j));
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t a0 = u4(R.v[2 * j], w), a1 = u4(R.v[2 * j + 1], w);
            const uint32_t plo = pair_lo(a0, a1), phi = pair_hi(a0, a1);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              o[h][2 * w] = dot2_bf16(pp[h], plo, o[h][2 * w]);
              o[h][2 * w + 1] = dot2_bf16(pp[h], phi, o[h][2 * w + 1]);
            }
          }
        }
      } else {
        // fp32 values take fp32 probabilities: broadcast them unrounded
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float pu = group_bcast_at<LPR>(p[h / 4], xpose_lane<TPL>(h % 4, u));
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(pu, __uint_as_float(u4(R.v[u], e)), o[h][e]);
          }
        }
      }
    }
  };

  // Scores, online softmax and P.V of block blk held in R; a block at or
  // past blk_end is empty (every row masked).
  auto compute = [&](int blk, const KvRegs<TPL>& R) {
    const int t0 = block_start(blk);
    int lo, hi;
    block_range(blk, t0, lo, hi);
    if (blk >= blk_end) hi = lo;
    // heads that attend this block (a union list names them; else all)
    uint32_t heads = 0xffu;
    if constexpr (SET == kSetUnion) heads = blk < n_sb ? (uint32_t)list[blk] >> 24 : 0xffu;
    if constexpr (kXpose) {
      compute_xpose(t0, lo, hi, heads, R);
      return;
    }
    // scores (log2 units) of the lane's TPL tokens
    float s[TPL][G];
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int t = t0 + u * RPI + r;
      const bool valid = t >= lo && t < hi;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float acc;
        if constexpr (BF16) {
          acc = dot2_bf16_first(R.k[u].x, qv[h].x);
          acc = dot2_bf16(R.k[u].y, qv[h].y, acc);
          acc = dot2_bf16(R.k[u].z, qv[h].z, acc);
          acc = dot2_bf16(R.k[u].w, qv[h].w, acc);
        } else {
          acc = __uint_as_float(R.k[u].x) * __uint_as_float(qv[h].x);
          acc = fmaf(__uint_as_float(R.k[u].y), __uint_as_float(qv[h].y), acc);
          acc = fmaf(__uint_as_float(R.k[u].z), __uint_as_float(qv[h].z), acc);
          acc = fmaf(__uint_as_float(R.k[u].w), __uint_as_float(qv[h].w), acc);
        }
        acc = row_sum<LPR>(acc) * a.scale_log2;
        s[u][h] = valid && ((heads >> h) & 1u) ? acc : NEG_INF;
      }
    }

    // online softmax with a lazily moved reference maximum
    float p[TPL][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int u = 1; u < TPL; ++u) mx = fmaxf(mx, s[u][h]);
      if (mx > m[h] + kTau) {
        const float alpha = fast_exp2(m[h] - mx);  // 0 when m was -inf
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] *= alpha;
        m[h] = mx;
      }
      const float mu = m[h] == NEG_INF ? 0.f : m[h];
      float ls = 0.f;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        p[u][h] = fast_exp2(s[u][h] - mu);
        ls += p[u][h];
      }
      l[h] += ls;
    }

    // P.V (a masked row has p = 0 and finite values: it adds nothing)
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < TPL; u += 2) {
        uint32_t pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pp[h] = pack_bf16x2(p[u][h], p[u + 1][h]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = u4(R.v[u], w), a1 = u4(R.v[u + 1], w);
          const uint32_t plo = pair_lo(a0, a1), phi = pair_hi(a0, a1);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            o[h][2 * w] = dot2_bf16(pp[h], plo, o[h][2 * w]);
            o[h][2 * w + 1] = dot2_bf16(pp[h], phi, o[h][2 * w + 1]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(p[u][h], __uint_as_float(u4(R.v[u], e)), o[h][e]);
      }
    }
  };

  // One block per wave step: its page (a scalar load) is looked up one step
  // ahead; the waves of the CU overlap each other's loads and arithmetic.
  const bool paged_lookup = PAGED_FAST && pt;
  int blk = __builtin_amdgcn_readfirstlane(blk_begin + wave);
  int ph = paged_lookup && blk < blk_end ? page_of(blk) : 0;
  if constexpr (gqa_double_buffer<BF16, G>()) {
    // With two waves per SIMD a wave's arithmetic would leave its SIMD with
    // little in flight: the next block's loads go out before this block's
    // arithmetic, into the other buffer.
    // Every step issues its loads unconditionally (past the wave's last
    // block it loads that block again, from L2) so that the wait before
    // each block's arithmetic counts only the other buffer's loads.
    KvRegs<TPL> R0, R1;
    if (blk < blk_end) {
      int ph1 = ph;
      issue(blk, ph, R0);
      if (paged_lookup && blk + kWaves < blk_end) ph1 = page_of(blk + kWaves);
      for (;;) {
        const int b1 = blk + kWaves < blk_end ? blk + kWaves : blk;
        int ph2 = ph1;
        issue(b1, ph1, R1);
        if (paged_lookup && b1 + kWaves < blk_end) ph2 = page_of(b1 + kWaves);
        compute(blk, R0);
        if (b1 == blk) break;
        const int b2 = b1 + kWaves < blk_end ? b1 + kWaves : b1;
        ph1 = ph2;
        issue(b2, ph2, R0);
        if (paged_lookup && b2 + kWaves < blk_end) ph1 = page_of(b2 + kWaves);
        compute(b1, R1);
        if (b2 == b1) break;
        blk = b2;
      }
    }
  } else {
    for (; blk < blk_end; blk += kWaves) {
      KvRegs<TPL> R;
      issue(blk, ph, R);
      if (paged_lookup && blk + kWaves < blk_end) ph = page_of(blk + kWaves);
      compute(blk, R);
    }
  }

  if constexpr (kXpose) {  // each head's denominator, in every lane of the row
#pragma unroll
    for (int k = 0; k < kNB; ++k) {
      float ls = lc[k] + dpp_f32<0xB1>(lc[k]);
      if constexpr (TPL == 4) ls += dpp_f32<0x4E>(ls);
#pragma unroll
      for (int i = 0; i < 4; ++i) l[4 * k + i] = group_bcast_at<LPR>(ls, xpose_lane<TPL>(i, 0));
    }
  }

  // merge the token rows of the wave (lanes c, c + LPR, ...)
#pragma unroll
  for (int d = LPR; d < 64; d <<= 1) {
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

  const size_t row0 = (size_t)b * a.Hq + (size_t)qh0;
  // an explicit sink logit joins the denominator once per row: here when
  // this workgroup holds the whole row, else in the combine
  const bool with_sink = a.sink != nullptr && a.num_splits == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    const float sink2 = with_sink ? a.sink[qh0 + h] * kLog2e : NEG_INF;
    M = fmaxf(M, sink2);
    const float mu = M == NEG_INF ? 0.f : M;
    float lsum = with_sink ? fast_exp2(sink2 - mu) : 0.f, acc = 0.f;
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
    case 1: launch_kernel(gqa_split_kernel<BF16, D, 1, FAST>, grid, block, s, a); break;
    case 2: launch_kernel(gqa_split_kernel<BF16, D, 2, FAST>, grid, block, s, a); break;
    case 4: launch_kernel(gqa_split_kernel<BF16, D, 4, FAST>, grid, block, s, a); break;
    case 8: launch_kernel(gqa_split_kernel<BF16, D, 8, FAST>, grid, block, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_d(const GqaArgs& a, hipStream_t s) {
  const bool fast = !a.page_table || a.page_size % kStep == 0;
  if (a.block_list) {  // listed 16-token blocks: the page table (or contiguous cache) is block-aligned
    if (!fast) return hipErrorInvalidValue;
    if (!a.list_count) {
      dim3 grid(a.num_splits, a.Hq, a.B), block(kThreads);
      launch_kernel(gqa_split_kernel<BF16, D, 1, true, kSetPerHead>, grid, block, s, a);
      return hipGetLastError();
    }
    dim3 grid(a.num_splits, a.Hkv, a.B), block(kThreads);
    switch (a.G) {
      case 1: launch_kernel(gqa_split_kernel<BF16, D, 1, true, kSetUnion>, grid, block, s, a); break;
      case 2: launch_kernel(gqa_split_kernel<BF16, D, 2, true, kSetUnion>, grid, block, s, a); break;
      case 4: launch_kernel(gqa_split_kernel<BF16, D, 4, true, kSetUnion>, grid, block, s, a); break;
      case 8: launch_kernel(gqa_split_kernel<BF16, D, 8, true, kSetUnion>, grid, block, s, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return fast ? launch_df<BF16, D, true>(a, s) : launch_df<BF16, D, false>(a, s);
}

// Resident split-kernel workgroups per CU, queried once per kernel variant.
template <bool BF16, int D, int G, bool FAST>
int occupancy_one() {
  static const int n = [] {
    int v = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gqa_split_kernel<BF16, D, G, FAST>, kThreads, 0) ==
                   hipSuccess
               ? v
               : 0;
  }();
  return n;
}

template <bool BF16, int D, int G, int SET>
int occupancy_listed() {
  static const int n = [] {
    int v = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gqa_split_kernel<BF16, D, G, true, SET>, kThreads,
                                                        0) == hipSuccess
               ? v
               : 0;
  }();
  return n;
}

template <bool BF16, int D>
int occupancy_set(int G, bool uni) {
  if (!uni) return occupancy_listed<BF16, D, 1, kSetPerHead>();
  switch (G) {
    case 1: return occupancy_listed<BF16, D, 1, kSetUnion>();
    case 2: return occupancy_listed<BF16, D, 2, kSetUnion>();
    case 4: return occupancy_listed<BF16, D, 4, kSetUnion>();
    case 8: return occupancy_listed<BF16, D, 8, kSetUnion>();
    default: return 0;
  }
}

template <bool BF16, int D, bool FAST>
int occupancy_g(int G) {
  switch (G) {
    case 1: return occupancy_one<BF16, D, 1, FAST>();
    case 2: return occupancy_one<BF16, D, 2, FAST>();
    case 4: return occupancy_one<BF16, D, 4, FAST>();
    case 8: return occupancy_one<BF16, D, 8, FAST>();
  }
  return 0;
}

// Merge split partials (o_j normalised, lse_j in log2 units):
// lse = max + log2 sum_j 2^(lse_j - max); o = sum_j 2^(lse_j - lse) o_j.
// One thread per four consecutive output elements of a row; it loads its
// row's split log-sum-exps and its 16-byte pieces of the split partials
// together (one memory round trip), then merges.  Splits may also hand over
// unnormalised sums with their reference maximum and softmax denominator
// (CombineArgs::part_l): the same merge with weights 2^(m - M) on both the
// sums and the denominators.
constexpr int kCombineThreads = 256;
constexpr int kMaxCombineSplits = 256;
constexpr int kCombineChunk = 16;

template <bool BF16>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(const CombineArgs a) {
  const float NEG_INF = -__builtin_inff();
  const int D4 = a.D / 4;
  const size_t e = (size_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (e >= (size_t)a.rows * D4) return;
  const int row = (int)(e / D4), d = 4 * (int)(e % D4);
  // this row's partials: entries base .. base + S - 1
  int S = a.splits;
  size_t base = (size_t)row * S;
  const float* pl;
  const float* ps;
  const float4* po;
  auto at = [&](size_t bs) {
    pl = a.part_lse + bs;
    ps = a.part_l ? a.part_l + bs : nullptr;
    po = (const float4*)(a.part_o + bs * a.D + d);
  };
  float x[kCombineChunk], l[kCombineChunk];
  float4 v[kCombineChunk];
  auto load = [&](int j0) {
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const bool in = j0 + u < S;
      x[u] = in ? pl[j0 + u] : NEG_INF;
      v[u] = in ? po[(size_t)(j0 + u) * D4] : make_float4(0.f, 0.f, 0.f, 0.f);
      l[u] = ps && in ? ps[j0 + u] : 1.f;
    }
  };
  at(base);
  load(0);
  if (a.items) {
    // sequence b's items own rows first * heads .. + count * heads,
    // head-major.  The first loads above went to row * splits: where a plan
    // of full-length sequences (splits items each) puts them, the same
    // layout as the split grid; they are redone elsewhere.
    const int b = row / a.heads, h = row - b * a.heads;
    const int n = a.items[2 * b + 1];
    const size_t tb = (size_t)a.items[2 * b] * a.heads + (size_t)h * n;
    if (n != S || tb != base) {
      S = n;
      base = tb;
      at(base);
      load(0);
    }
  }
  float M = NEG_INF, wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < S; j0 += kCombineChunk) {
    if (j0 > 0) load(j0);
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) Mc = fmaxf(Mc, x[u]);
    const float mu = Mc == NEG_INF ? 0.f : Mc;
    const float f = fast_exp2(M - mu);  // rescales the running sums (0 while M is -inf)
    wsum *= f;
    acc.x *= f;
    acc.y *= f;
    acc.z *= f;
    acc.w *= f;
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const float w = fast_exp2(x[u] - mu);
      wsum = fmaf(w, l[u], wsum);
      acc.x = fmaf(w, v[u].x, acc.x);
      acc.y = fmaf(w, v[u].y, acc.y);
      acc.z = fmaf(w, v[u].z, acc.z);
      acc.w = fmaf(w, v[u].w, acc.w);
    }
    M = Mc;
  }
  if (a.sink) {  // one more term, exp(sink), with a zero value
    const float x = a.sink[row % a.sink_heads] * kLog2e;
    const float Mc = fmaxf(M, x);
    const float f = fast_exp2(M - Mc);  // 0 while M is -inf
    wsum = wsum * f + fast_exp2(x - Mc);
    acc.x *= f;
    acc.y *= f;
    acc.z *= f;
    acc.w *= f;
    M = Mc;
  }
  const float o0 = wsum > 0.f ? acc.x / wsum : 0.f, o1 = wsum > 0.f ? acc.y / wsum : 0.f;
  const float o2 = wsum > 0.f ? acc.z / wsum : 0.f, o3 = wsum > 0.f ? acc.w / wsum : 0.f;
  const size_t o = (size_t)row * a.D + d;
  if constexpr (BF16) {
    *(uint2*)((uint16_t*)a.out + o) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
  } else {
    *(float4*)((float*)a.out + o) = make_float4(o0, o1, o2, o3);
  }
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

int gqa_listed_blocks_per_cu(bool bf16, int D, int G, bool uni) {
  if (bf16) return D == 64 ? occupancy_set<true, 64>(G, uni) : occupancy_set<true, 128>(G, uni);
  return D == 64 ? occupancy_set<false, 64>(G, uni) : occupancy_set<false, 128>(G, uni);
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
  if (!a.items && a.splits > kMaxCombineSplits) return hipErrorInvalidValue;
  if (a.D % 4 != 0) return hipErrorInvalidValue;
  const size_t total = (size_t)a.rows * (a.D / 4);
  const unsigned blocks = (unsigned)((total + kCombineThreads - 1) / kCombineThreads);
  if (a.bf16) launch_kernel(lse_combine_kernel<true>, blocks, kCombineThreads, s, a);
  else launch_kernel(lse_combine_kernel<false>, blocks, kCombineThreads, s, a);
  return hipGetLastError();
}

}  // namespace dattn
