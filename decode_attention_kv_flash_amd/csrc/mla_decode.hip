// Absorbed MLA decode attention over a 576-wide latent cache, dense or over a
// gathered top-k token list (sparse MLA), on bf16 MFMA.
//
// Every query head reads the same latent row [c_KV (512) | k_pe (64)]
// ("Attention Optimizations", "DSA: DeepSeek Sparse Attention", "Computation
// Path"; with W_UK absorbed into the query, "Overview of Attention
// Mechanism", MLA), so the scores of a tile of tokens for many heads are one
// dense product, and so is P.c_KV.  A workgroup owns (sequence, 128 or 64
// heads, token split) and reads each latent row of its split once; each wave
// owns 32 heads, one wave per SIMD.
//
// Data movement.  Tiles of 16 rows (18 KB) go from HBM straight into LDS by
// direct-to-LDS loads (global_load_lds_dwordx4: no registers in between),
// into eight tile buffers: while one tile is P.V'd and the next scored, six
// more are in flight (108 KB per CU), enough to keep the HBM stream full.  A
// contiguous cache needs no lookup: a tile is 18 KB of consecutive rows, one
// uniform base address plus a fixed offset per lane.  A paged cache and a
// gathered list resolve their rows once into a row table in LDS.  Row r of a
// tile keeps its 16-byte chunk c at slot c ^ f(r) within its group of eight
// chunks, which makes both LDS read patterns below free of bank conflicts.
//
// Per tile (16 tokens), in one instruction stream per wave:
//   * S^T[token, head] = C[token, :] . Q^T over 576 dims for the wave's own 32
//     heads: 18 k-steps of two 16x16x32 bf16 MFMAs (two groups of 16 heads),
//     A = latent chunks from LDS (one read serves both), B = the wave's query
//     rows, held in registers for the whole split;
//   * online softmax in log2 units per head ("All the attentions", section 1:
//     running maximum and sum); the reference maximum is set by the head's
//     first scores and moves only when a score passes it by more than 2^64
//     (exponentials stay finite in fp32 and keep their relative precision);
//     when that happens the workgroup restarts the split with the larger
//     reference, so the accumulators are never rescaled.  P goes to LDS in
//     the A layout of the 32x32x16 MFMA (a head's 8 consecutive tokens per
//     lane), which one v_permlane16_swap per register pair makes from the
//     score layout;
//   * O[head, dims] += P . C[:, dims]: the wave owns 512 / W of the output
//     dims for all the workgroup's heads (W waves), 16 32x32x16 MFMAs; the B
//     operand (tokens x dims) comes from the row-major tile by the gfx950
//     transpose read ds_read_b64_tr_b16, so each wave reads only its own
//     dims of the value, and every head's P from the other waves through LDS.
// A single wave per SIMD issues at most one instruction every four cycles,
// so the stream is built to fit the matrix cores' time: the score MFMAs of
// tile t + 1, the P.V MFMAs of tile t - 1, the softmax of tile t and the
// copies of tile t + 6 are interleaved, each LDS operand read a few MFMA
// steps ahead of its use.
//
// O lives in accumulation registers (AGPRs) for the whole split.  All MFMAs
// are issued by inline assembly that pins each operand to its register file
// (O in AGPRs; scores, Q and the tile fragments in VGPRs) and carries the
// wait states the compiler would otherwise insert.  The tile copies are
// inline assembly too: the compiler then tracks the LDS reads alone and
// waits for each exactly, and the copies' completion is awaited explicitly
// before the barrier that hands a tile to the other waves.
// P is rounded to bf16 for the MFMA; everything else accumulates in fp32.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kDc = 512;            // c_KV width (the value)
constexpr int kDq = 576;            // latent row: c_KV + k_pe
constexpr int kRowBytes = kDq * 2;
constexpr int kChunks = kDq / 8;    // 16-byte chunks per row
constexpr int kTile = 16;           // tokens per tile
constexpr int kHeadsPerWave = 32;
constexpr int kTileChunks = kTile * kChunks;              // 1152
constexpr int kTileBytes = kTileChunks * 16;              // 18432
constexpr int kKSteps = kDq / 32;                         // 18 score k-steps of 32 dims
constexpr int kNTiles = kDc / 32;                         // 16 output tiles of 32 dims
constexpr int kRing = 3;                                  // LDS fragments in flight per operand
constexpr float kTau = 64.0f;                             // reference-maximum slack (log2)
constexpr float kTwoTau = 18446744073709551616.0f;         // 2^kTau
constexpr uint32_t kPad = 0x80000000u;                    // row-table flag: no token here
constexpr int kMaxTiles = kMlaMaxSplitTokens / kTile;
constexpr int kRowTable = (kMaxTiles + 1) * kTile;  // plus one tile of padding
static_assert(kMlaMaxSplitTokens % kTile == 0, "splits hold whole tiles");
// tile buffers: eight for a contiguous cache, seven beside a row table; tile
// t + kBuffers - 2 is copied into the buffer of tile t - 2 while tiles t - 1
// (P.V), t (softmax) and t + 1 (scores) are in use
template <bool TABLE> constexpr int kBuffersOf = TABLE ? 7 : 8;
constexpr int kPBytes = 4 * 1024;  // P of one tile for up to 128 heads, bf16
static_assert(8 * kTileBytes + 2 * kPBytes + 64 <= 160 * 1024, "fits the LDS");
static_assert(7 * kTileBytes + 2 * kPBytes + kRowTable * 4 + ((kMaxTiles + 32) / 32) * 4 + 64 <= 160 * 1024,
              "fits the LDS");

// Chunk permutation of row r (low three bits of the chunk index only): the
// 16-byte chunk c of tile row r sits at slot c ^ f(r) of its group of eight.
// Both read patterns must be free of LDS bank conflicts: the score reads
// (lane l: row l % 16, chunk 4 ks + l / 16, 16 bytes) and the transpose
// reads (lane l: rows 8 (l / 32) + (l % 16) / 4 and + 4, chunks 4 n + 0..3,
// 8 bytes).  f was chosen by measurement: among all 4096 XOR-linear maps of
// r's four bits to three, the rocprofv3 counter SQ_LDS_BANK_CONFLICT on
// gfx950 reads zero for both patterns only when bit 1 of r flips bit 2 of the
// slot (the map here also lets bit 2 of r flip bit 1); the swizzle of the
// earlier 32-row tile left the score reads 2-way conflicted.
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1);
}

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;

// One wave-wide 16-byte-per-lane copy into LDS at lds_dst + 16 * lane, from
// sbase + voff (sbase uniform, in SGPRs) or from a per-lane address.  M0
// carries the LDS address; it is declared clobbered (the compiler keeps
// nothing in it across the copy) rather than saved and restored.
__device__ __forceinline__ void copy_to_lds_sv(uint32_t voff, const void* sbase, uint32_t lds_dst) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds_dst)
      : "memory", "m0");
}

__device__ __forceinline__ void copy_to_lds_v(const void* src, uint32_t lds_dst) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      :
      : "v"((uint64_t)(uintptr_t)src), "s"(lds_dst)
      : "memory", "m0");
}

// Maxima of values the compiler cannot prove canonical (MFMA results): as
// plain v_max instructions, without the canonicalising v_max x, x it would
// put before each operand.
__device__ __forceinline__ float max2(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float max3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

// The O accumulators are written by MFMAs the compiler does not see; before
// ordinary code reads or writes them, let the last of those MFMAs retire
// (more than the 18 wait states a 32x32 MFMA result needs) and make every
// later access depend on this point.
__device__ __forceinline__ void settle(f32x16_t (&acc)[kNTiles]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
#pragma unroll
  for (int n = 0; n < kNTiles; ++n) asm volatile("" : "+a"(acc[n]));
}

// Barrier with the newest k tiles' copies (of kc copies each) still in flight.
template <int kc>
__device__ __forceinline__ void barrier_tiles_in_flight(int k) {
  switch (k) {
    case 0: barrier_in_flight<0>(); break;
    case 1: barrier_in_flight<kc>(); break;
    case 2: barrier_in_flight<2 * kc>(); break;
    case 3: barrier_in_flight<3 * kc>(); break;
    case 4: barrier_in_flight<4 * kc>(); break;
    case 5: barrier_in_flight<5 * kc>(); break;
    default: barrier_in_flight<6 * kc>(); break;
  }
}

// TABLE: rows through the LDS row table (a paged cache, or SPARSE lists);
// otherwise a contiguous cache, whose tiles are consecutive rows.
template <bool SPARSE, bool TABLE, int NW>
__global__ __launch_bounds__(64 * NW, 1) void mla_split_kernel(const MlaArgs a) {
  constexpr int kThreads = 64 * NW;
  constexpr int kBuffers = kBuffersOf<TABLE>;
  constexpr int kAhead = kBuffers - 2;                   // tiles requested ahead
  constexpr int kPerWave = kTileChunks / NW;             // 16-byte slots one wave copies per tile
  constexpr int kCopies = (kPerWave + 63) / 64;          // copy instructions per wave and tile
  constexpr int kLastLanes = kPerWave - 64 * (kCopies - 1);  // lanes of the last one
  constexpr int kCopyStride = kKSteps / kCopies;          // k-steps between two copies
  constexpr int kHG = NW;                                // 32-head groups of the workgroup
  constexpr int kNT = kNTiles / NW;                      // 32-dim output tiles of one wave
  constexpr int kPStart = kKSteps - kHG * kNT;           // first k-step with a P.V MFMA
  static_assert(kTileChunks % NW == 0 && kLastLanes > 0 && kLastLanes <= 64, "copy split");
  static_assert(kCopyStride >= 1 && kPStart >= 1, "fits the k-steps");
  static_assert(!SPARSE || TABLE, "gathered rows go through the row table");
  const float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(16))) char tiles[kBuffers * kTileBytes];
  // P of two consecutive tiles for all heads, each in the 32x32x16 A layout:
  // head group hg at [hg][lane] (16 bytes)
  __shared__ __attribute__((aligned(16))) char pbuf[2][kPBytes];
  __shared__ __attribute__((aligned(16))) uint32_t rows[TABLE ? kRowTable : 4];
  __shared__ int first_valid;
  // bit t: tile t holds a position without a token (its scores need the mask)
  __shared__ uint32_t tile_pad[TABLE ? (kMaxTiles + 32) / 32 : 1];
  // restart votes: iteration u votes in slot u % 3, every wave reads it after
  // the iteration's barrier, and iteration u + 2 clears it, so a fast wave
  // never touches a vote a slow wave has yet to read
  __shared__ int restart_vote[3];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g4 = lane >> 4, half = lane >> 5;
  // grid (B, splits, head blocks): the sequence index fastest, so that the
  // workgroups of one sequence share an XCD and its L2 (B a multiple of 8)
  const int b = blockIdx.x;
  const int split = blockIdx.y;
  const int hw = blockIdx.z * (NW * kHeadsPerWave);   // the workgroup's first head
  const int h0 = hw + wave * kHeadsPerWave;           // this wave's score heads
  const int d0 = wave * (kDc / NW);                   // this wave's output dims

  int N;
  if constexpr (SPARSE) {
    N = a.k_sel;
  } else {
    const int cap = a.page_table ? a.page_size * a.max_pages : a.S_max;
    N = max(0, min(a.seq_lens[b], cap));
  }
  const int per = ((N + a.num_splits - 1) / a.num_splits + kTile - 1) / kTile * kTile;
  const int f_begin = min(N, split * per);
  const int f_end = min(N, f_begin + per);
  const int n_tok = f_end - f_begin;
  int n_tiles = min((n_tok + kTile - 1) / kTile, kMaxTiles);

  // TABLE: the source of each position of the split (a token index of the
  // list, or a page of the table), for the first kPre positions of this
  // thread; requested before the query rows so that the two round trips
  // overlap.  -1: no token.
  constexpr int kPre = 2;
  // positions of the split plus one all-padding tile (none for an empty split,
  // which reads nothing)
  const int n_rows = TABLE && n_tiles > 0 ? (n_tiles + 1) * kTile : 0;
  auto entry_src = [&](int i) -> int {
    const int f = f_begin + i;
    if constexpr (SPARSE) {
      return f < f_end ? a.idx[(size_t)b * a.k_sel + f] : -1;
    } else {
      const int t = f < f_end ? f : f_end - 1;
      return a.page_table[(size_t)b * a.max_pages + (t >> a.log2_page)];
    }
  };
  int pre[kPre];
  if constexpr (TABLE) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int i = (int)threadIdx.x + u * kThreads;
      pre[u] = i < n_rows ? entry_src(i) : -1;
    }
  }

  // Q^T fragments (B operand of the 16x16x32 scores): for head group hh the
  // lane holds head h0 + 16 hh + l16, dims 32 ks + 8 g4 + [0, 8)
  bf16x8_t qf[kKSteps][2];
  {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint16_t* qrow = a.q + ((size_t)b * a.H + h0 + 16 * hh + l16) * kDq + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks][hh] = *(const bf16x8_t*)(qrow + 32 * ks);
    }
  }

  if (threadIdx.x == 0) {
    first_valid = 0x7fffffff;
    restart_vote[0] = restart_vote[1] = restart_vote[2] = 0;
  }
  // ---- row table: cache row of every position of the split and of one
  // all-padding tile past it.  Flag kPad marks a position without a token;
  // its entry still names a row of finite data (a real row of the same
  // split), so that P = 0 times it stays 0.
  // The barriers of the set-up wait for LDS only: the query rows stay in
  // flight under the table's construction and the first copies.
  if constexpr (TABLE) {
    if (threadIdx.x < (kMaxTiles + 32) / 32) tile_pad[threadIdx.x] = 0u;
    barrier_in_flight<63>();
    int fv = 0x7fffffff;  // this thread's first position with a token (SPARSE)
    auto place = [&](int i, int src) {
      const int f = f_begin + i;
      uint32_t e;
      if constexpr (SPARSE) {
        const bool ok = src >= 0 && src < a.S_max;
        e = ok ? (uint32_t)b * (uint32_t)a.S_max + (uint32_t)src : kPad;
        if (ok) fv = min(fv, i);
      } else {
        const bool ok = f < f_end;
        const int t = ok ? f : f_end - 1;
        const uint32_t row = (uint32_t)src * (uint32_t)a.page_size + (uint32_t)(t & (a.page_size - 1));
        e = row | (ok ? 0u : kPad);
      }
      rows[i] = e;
      if (e & kPad) atomicOr(&tile_pad[(i / kTile) >> 5], 1u << ((i / kTile) & 31));
    };
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int i = (int)threadIdx.x + u * kThreads;
      if (i < n_rows) place(i, pre[u]);
    }
    for (int i = (int)threadIdx.x + kPre * kThreads; i < n_rows; i += kThreads) place(i, entry_src(i));
    if constexpr (SPARSE) {
      // the workgroup's first position with a token: a minimum per wave,
      // then one LDS atomic per wave
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) fv = min(fv, __shfl_xor(fv, d));
      if (lane == 0 && fv != 0x7fffffff) atomicMin(&first_valid, fv);
    }
    barrier_in_flight<63>();
    if constexpr (SPARSE) {
      const int fvw = first_valid;
      if (fvw == 0x7fffffff) {
        n_tiles = 0;  // nothing to attend in this split
      } else {
        const uint32_t fb = rows[fvw] | kPad;
        for (int i = threadIdx.x; i < n_rows; i += kThreads)
          if (rows[i] == kPad) rows[i] = fb;
        barrier_in_flight<63>();
      }
    }
  } else {
    barrier_in_flight<63>();
  }

  const uint32_t tiles_base = lds_address(tiles);
  // buffer of tile tix >= -1
  auto buffer = [&](int tix) -> uint32_t {
    return tiles_base + (uint32_t)((tix + kBuffers) % kBuffers) * kTileBytes;
  };
  const uint32_t pbuf_base = lds_address(pbuf);

  // ---- tile copy: this wave's copy j fills slots kPerWave * wave + 64 j +
  // lane; slot q of a tile is row q / 72, stored chunk q % 72, i.e. logical
  // chunk (q % 72) ^ f(row).  The lane's (row, chunk) of each copy is fixed.
  // row | logical chunk << 8 of copy j, two 16-bit entries per register
  uint32_t rc2[(kCopies + 1) / 2];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const uint32_t q = (uint32_t)(kPerWave * wave + 64 * j + lane);
    const uint32_t r = q / kChunks, cs = q - r * kChunks;
    const uint32_t c = (cs & ~7u) | ((cs & 7u) ^ (uint32_t)swz((int)r));
    if (j % 2 == 0) rc2[j / 2] = r | (c << 8);
    else rc2[j / 2] |= (r | (c << 8)) << 16;
  }
  auto rc = [&](int j) -> uint32_t { return j % 2 == 0 ? rc2[j / 2] & 0xffffu : rc2[j / 2] >> 16; };
  const char* latent = (const char*)a.latent;
  // Per tile: the copies' sources.  TABLE: each lane's row from the table
  // (read ahead of the copies, so that no LDS wait lands among the operand
  // reads); otherwise a uniform base and each lane's offset, rows past the
  // split end re-reading its last row (finite data; their P is 0).
  struct CopySrc {
    uint32_t v[kCopies];
    const char* base;
  };
  auto copy_src = [&](int tix) -> CopySrc {
    CopySrc c;
    if constexpr (TABLE) {
      const uint32_t* rt = rows + tix * kTile;
#pragma unroll
      for (int j = 0; j < kCopies; ++j) c.v[j] = rt[rc(j) & 0xff] & ~kPad;
      c.base = latent;
    } else {
      c.base = latent + ((size_t)b * a.S_max + f_begin + tix * kTile) * kRowBytes;
      const uint32_t last = (uint32_t)(min(kTile, n_tok - tix * kTile) - 1);
#pragma unroll
      for (int j = 0; j < kCopies; ++j) c.v[j] = min(rc(j) & 0xff, last) * kRowBytes + (rc(j) >> 8) * 16;
    }
    return c;
  };
  // copy j of tile tix: one wave-wide instruction (the last may use part of the wave)
  auto copy = [&](int tix, int j, const CopySrc& c) {
    const uint32_t dst = buffer(tix) + 16u * (uint32_t)(kPerWave * wave) + 1024u * j;
    if (j == kCopies - 1 && lane >= kLastLanes) return;
    if constexpr (TABLE) copy_to_lds_v(c.base + ((size_t)c.v[j] * kChunks + (rc(j) >> 8)) * 16, dst);
    else copy_to_lds_sv(c.v[j], c.base, dst);
  };
  auto issue = [&](int tix) {
    const CopySrc c = copy_src(tix);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) copy(tix, j, c);
  };

  // ---- per-lane parts of the LDS read patterns
  // scores (A of the 16x16x32): row l16, chunk 4 ks + g4
  const int sw_s = swz(l16);
  // P.V (B of the 32x32x16 via the transpose read): rows 8 half + (l16 >> 2)
  // (+ 4 for the second read), chunk d0 / 8 + 4 nt + 2 (g4 & 1) + ((l16 >> 1)
  // & 1), byte 8 (l16 & 1) within it
  const int rv = 8 * half + (l16 >> 2);
  const int cv = 2 * (g4 & 1) + ((l16 >> 1) & 1);
  const int sw_v0 = swz(rv), sw_v1 = swz(rv + 4);

  // O accumulators acc[hg * kNT + nt]: heads hw + 32 hg + .., dims d0 + 32 nt
  // + ..  Defined (zeroed) by MFMAs with zero operands, so that they are born
  // in AGPRs and never pass through VGPRs.
  f32x16_t acc[kNTiles];
  auto zero_acc = [&]() {
    const bf16x8_t z = {};
#pragma unroll
    for (int n = 0; n < kNTiles; ++n)
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc[n]) : "v"(z));
  };
  zero_acc();
  // per head group hh (head h0 + 16 hh + l16): m_run the reference maximum
  // (log2 units), m_seen the largest score so far, l_run this lane's share
  // of the softmax denominator
  float m_run[2] = {NEG_INF, NEG_INF}, m_seen[2] = {NEG_INF, NEG_INF}, l_run[2] = {0.f, 0.f};
  // S^T of the tile whose softmax comes next: for group hh the lane holds
  // head 16 hh + l16, tokens 4 g4 + [0, 4)
  f32x4_t sc[2];

  // The tile pipeline.  Iteration t (0 <= t <= n_tiles) runs, interleaved
  // on one instruction stream:
  //   S: the score MFMAs of tile t + 1 (buffer t + 1),
  //   X: the softmax of tile t (its scores from iteration t - 1) -> its P to
  //      pbuf[t % 2],
  //   P: the P.V MFMAs of tile t - 1 (buffer t - 1, P from pbuf[(t - 1) % 2]),
  //   C: the copies of tile t + kAhead into the buffer tile t - 2 freed.
  // The first and last iterations run the same stream on stand-ins: tile -1
  // has P = 0 (a zeroed P buffer; its tile buffer holds finite data), and
  // tile n_tiles is all padding (its scores are dropped, its softmax changes
  // nothing).
  auto stream = [&](auto with_copies, int t, int slot) {
    constexpr bool copies = decltype(with_copies)::value;
    const uint32_t sbuf = buffer(t + 1), vbuf = buffer(t - 1);
    const uint32_t pin = pbuf_base + (uint32_t)((t + 1) & 1) * kPBytes;  // P of tile t - 1
    const uint32_t pout = pbuf_base + (uint32_t)(t & 1) * kPBytes + 16u * (uint32_t)(wave * 64 + lane);
    uint32_t so[2], vo[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      so[j] = sbuf + l16 * kRowBytes + 16 * ((4 * j + g4) ^ sw_s);
      const int cb = d0 / 8;  // 8 (d0 / 64) + 0: the wave's dims start on an 8-chunk group
      vo[j] = vbuf + rv * kRowBytes + 16 * (cb + ((4 * j + cv) ^ sw_v0)) + 8 * (l16 & 1);
      vo[2 + j] = vbuf + (rv + 4) * kRowBytes + 16 * (cb + ((4 * j + cv) ^ sw_v1)) + 8 * (l16 & 1);
      asm volatile("" : "+v"(so[j]), "+v"(vo[j]), "+v"(vo[2 + j]));
    }
    auto aread = [&](int k) -> bf16x8_t {  // chunk 4 k + g4 = 8 (k / 2) + (4 (k % 2) + g4)
      return *(const lds_bf16x8*)(uintptr_t)(so[k & 1] + 128 * (k >> 1));
    };
    auto vread = [&](int nt) -> bf16x8_t {  // chunk d0 / 8 + 4 nt + cv
      const uint32_t imm = 128 * (nt >> 1);
      const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(vo[nt & 1] + imm));
      const bf16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(vo[2 + (nt & 1)] + imm));
      return __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // X's inputs: padding of tile t; the copies' sources of tile t + kAhead
    bool pad[4] = {false, false, false, false};
    bool padded;
    if constexpr (TABLE) {
      padded = (tile_pad[t >> 5] >> (t & 31)) & 1u;
      const uint4 e = *(const uint4*)(rows + t * kTile + 4 * g4);
      pad[0] = e.x & kPad; pad[1] = e.y & kPad; pad[2] = e.z & kPad; pad[3] = e.w & kPad;
    } else {
      padded = t * kTile + kTile > n_tok;
#pragma unroll
      for (int i = 0; i < 4; ++i) pad[i] = t * kTile + 4 * g4 + i >= n_tok;
    }
    CopySrc csrc;
    if constexpr (copies) csrc = copy_src(t + kAhead);

    // P of tile t - 1 for every head group, and the first value fragments
    bf16x8_t pa[kHG];
#pragma unroll
    for (int hg = 0; hg < kHG; ++hg) pa[hg] = *(const lds_bf16x8*)(uintptr_t)(pin + 16u * (hg * 64 + lane));
    bf16x8_t ar[kRing], vr[2];
#pragma unroll
    for (int j = 0; j < kRing; ++j) ar[j] = aread(j);
    vr[0] = vread(0);
    vr[1] = vread(1);

    f32x4_t sn[2];
    float m4[2], mx[2], nmu[2], pe[2][4];
    uint32_t pk[2][2];
#pragma unroll
    for (int i = 0; i < kKSteps; ++i) {
      // S: scores of tile t + 1, k-step i, both head groups
      if (i == 0) {
        asm volatile("s_nop 2\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(sn[0]) : "v"(ar[0]), "v"(qf[0][0]));
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(sn[1]) : "v"(ar[0]), "v"(qf[0][1]));
      } else {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(sn[0]) : "v"(ar[i % kRing]), "v"(qf[i][0]));
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(sn[1]) : "v"(ar[i % kRing]), "v"(qf[i][1]));
      }
      if (i + kRing < kKSteps) ar[i % kRing] = aread(i + kRing);
      // P: P.V of tile t - 1, one (output tile, head group) per k-step from kPStart
      if (i >= kPStart) {
        const int u = i - kPStart, nt = u / kHG, hg = u % kHG;
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(acc[hg * kNT + nt]) : "v"(pa[hg]), "v"(vr[nt & 1]));
        if (hg == kHG - 1 && nt + 2 < kNT) vr[nt & 1] = vread(nt + 2);
      }
      // X: softmax of tile t, one piece per k-step
      if (i == 0) {
        if (padded) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (pad[q]) sc[0][q] = sc[1][q] = NEG_INF;
        }
      } else if (i == 1) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) m4[hh] = max3(sc[hh][0], sc[hh][1], max2(sc[hh][2], sc[hh][3]));
      } else if (i == 2) {
        // the head's 16 tokens are on the four lanes l16 + 16 g
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(m4[hh]), __float_as_uint(m4[hh]), false, false);
          m4[hh] = max2(__uint_as_float(w[0]), __uint_as_float(w[1]));
        }
      } else if (i == 3) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(m4[hh]), __float_as_uint(m4[hh]), false, false);
          mx[hh] = max2(__uint_as_float(w[0]), __uint_as_float(w[1])) * a.scale_log2;
        }
      } else if (i == 4) {
        // a head's first scores set its reference (its O is still zero); a
        // later score past the reference by more than kTau asks for a restart
        bool jump = false;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          m_seen[hh] = max2(m_seen[hh], mx[hh]);
          jump |= mx[hh] > m_run[hh] + kTau && m_run[hh] != NEG_INF;
          m_run[hh] = m_run[hh] == NEG_INF ? mx[hh] : m_run[hh];
          nmu[hh] = m_run[hh] == NEG_INF ? 0.f : -m_run[hh];
        }
        if (jump) restart_vote[slot] = 1;
      } else if (i >= 5 && i < 9) {
        const int hh = (i - 5) >> 1, q0 = 2 * ((i - 5) & 1);
        pe[hh][q0] = fast_exp2(__builtin_fmaf(sc[hh][q0], a.scale_log2, nmu[hh]));
        pe[hh][q0 + 1] = fast_exp2(__builtin_fmaf(sc[hh][q0 + 1], a.scale_log2, nmu[hh]));
      } else if (i == 9) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          l_run[hh] += (pe[hh][0] + pe[hh][1]) + (pe[hh][2] + pe[hh][3]);
          pk[hh][0] = pack_bf16x2(pe[hh][0], pe[hh][1]);
          pk[hh][1] = pack_bf16x2(pe[hh][2], pe[hh][3]);
        }
      } else if (i == 10) {
        // to the A layout of P.V: lane l takes head l % 32 and tokens
        // 8 (l / 32) + [0, 8) -- rows 0 and 1 (2 and 3) of 16 lanes trade
        // the group they do not keep -- and out to LDS for every wave
        const auto x0 = __builtin_amdgcn_permlane16_swap(pk[0][0], pk[1][0], false, false);
        const auto x1 = __builtin_amdgcn_permlane16_swap(pk[0][1], pk[1][1], false, false);
        uint4 v;
        v.x = x0[0];  // tokens 8 half + 0, 1
        v.y = x1[0];  // + 2, 3
        v.z = x0[1];  // + 4, 5
        v.w = x1[1];  // + 6, 7
        *(lds_bf16x8*)(uintptr_t)pout = __builtin_bit_cast(bf16x8_t, v);
      }
      // C: copies of tile t + kAhead spread over the k-steps
      if constexpr (copies) {
        if (i % kCopyStride == 0 && i / kCopyStride < kCopies) copy(t + kAhead, i / kCopyStride, csrc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ordinary code reads the scores next: let the last MFMA retire first
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sn[0]), "+v"(sn[1]));
    sc[0] = sn[0];
    sc[1] = sn[1];
  };

  // stand-ins for tile -1: zero P, finite values in its tile buffer
  auto zero_standins = [&]() {
    uint4* z = (uint4*)(tiles + (kBuffers - 1) * kTileBytes);
    for (int i = threadIdx.x; i < kTileBytes / 16; i += kThreads) z[i] = make_uint4(0u, 0u, 0u, 0u);
    uint4* zp = (uint4*)pbuf[1];
    for (int i = threadIdx.x; i < kPBytes / 16; i += kThreads) zp[i] = make_uint4(0u, 0u, 0u, 0u);
  };

  // Prologue: tiles 0..kAhead - 1 requested, tile 0 scored, tile 1 complete.
  auto prime = [&]() {
    zero_standins();
    const int first = min(n_tiles, kAhead);
    for (int t = 0; t < first; ++t) issue(t);
    barrier_tiles_in_flight<kCopies>(first - 1);  // tile 0 complete
    {
      const uint32_t sbuf = buffer(0);
      uint32_t so[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        so[j] = sbuf + l16 * kRowBytes + 16 * ((4 * j + g4) ^ sw_s);
        asm volatile("" : "+v"(so[j]));
      }
      auto aread = [&](int k) -> bf16x8_t {
        return *(const lds_bf16x8*)(uintptr_t)(so[k & 1] + 128 * (k >> 1));
      };
      bf16x8_t ar[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) ar[j] = aread(j);
#pragma unroll
      for (int i = 0; i < kKSteps; ++i) {
        if (i == 0) {
          asm volatile("s_nop 2\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(sc[0]) : "v"(ar[0]), "v"(qf[0][0]));
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(sc[1]) : "v"(ar[0]), "v"(qf[0][1]));
        } else {
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(sc[0]) : "v"(ar[i % kRing]), "v"(qf[i][0]));
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(sc[1]) : "v"(ar[i % kRing]), "v"(qf[i][1]));
        }
        if (i + kRing < kKSteps) ar[i % kRing] = aread(i + kRing);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sc[0]), "+v"(sc[1]));
    barrier_tiles_in_flight<kCopies>(max(first - 2, 0));  // tile 1 complete, stand-ins zeroed
  };

  // Iteration t of the pipeline above, then a barrier after which tile t + 2
  // is complete in LDS and tile t's P in pbuf for every wave (only the copies
  // of later tiles may be in flight), and the buffer of tile t - 1 is free.
  // A restart leaves the loop and runs the prologue again.
  while (n_tiles > 0) {
    prime();
    int slot = 0;
    bool again = false;
    // while tiles remain to be requested (copies in every iteration), then the tail
    const int n_copying = max(n_tiles - kAhead, 0);
    int t = 0;
    for (; t < n_copying; ++t) {
      if (threadIdx.x == 0) restart_vote[slot == 2 ? 0 : slot + 1] = 0;  // iteration t - 2's
      stream(std::true_type{}, t, slot);
      barrier_in_flight<(kAhead - 2) * kCopies>();  // tiles t + 3 .. t + kAhead in flight
      if (restart_vote[slot]) {
        again = true;
        break;
      }
      slot = slot == 2 ? 0 : slot + 1;
    }
    if (!again) {
      for (; t <= n_tiles; ++t) {
        if (threadIdx.x == 0) restart_vote[slot == 2 ? 0 : slot + 1] = 0;
        stream(std::false_type{}, t, slot);
        barrier_tiles_in_flight<kCopies>(min(max(n_tiles - 1 - (t + 2), 0), kAhead - 2));
        if (restart_vote[slot]) {
          again = true;
          break;
        }
        slot = slot == 2 ? 0 : slot + 1;
      }
    }
    if (!again) break;
    // some head's maximum jumped: redo the split with every head's reference
    // at the largest score it has seen (each restart raises a reference by
    // more than kTau, so restarts are few)
    barrier_in_flight<0>();  // every wave has read the vote; no copy in flight
    if (threadIdx.x == 0) restart_vote[0] = restart_vote[1] = restart_vote[2] = 0;
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);  // in-flight MFMAs retire first
    zero_acc();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      m_run[hh] = m_seen[hh];
      l_run[hh] = 0.f;
    }
  }
  settle(acc);

  // unnormalised partials: O (relative to m_run), m_run and l per head; the
  // combine merges the splits and divides
  float l_tot[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run[hh]), __float_as_uint(l_run[hh]),
                                                      false, false);
    const float x = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);
    const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    l_tot[hh] = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
  }
  const size_t roww = (size_t)b * a.H + hw;
  const int lj = lane & 31;
#pragma unroll
  for (int hg = 0; hg < kHG; ++hg)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        a.part_o[((roww + 32 * hg + 8 * (v / 4) + 4 * half + (v % 4)) * a.num_splits + split) * kDc + d0 +
                 32 * nt + lj] = acc[hg * kNT + nt][v];
  if (g4 == 0) {
    const size_t row0 = (size_t)b * a.H + h0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const size_t r = (row0 + 16 * hh + l16) * a.num_splits + split;
      a.part_lse[r] = l_tot[hh] > 0.f ? m_run[hh] : NEG_INF;
      a.part_l[r] = l_tot[hh];
    }
  }
}

// ---------------------------------------------------------------------------
// The 32-row kernel (128 heads per workgroup; rows from a contiguous cache
// [B, S_max, 576], a sparse list, or a paged cache with pages of at least 8
// rows): tiles of 32 rows and 32x32x16 MFMAs throughout.  A 32x32x16 MFMA
// keeps the matrix core busy for 32 cycles, in which the wave can issue
// a few other instructions; with 16x16x32 scores there is half that room per
// instruction.  So here every k-step of the scores is one MFMA for the
// wave's 32 heads, and the softmax, the operand reads and the copies fit
// between the MFMAs.
//
// Per tile t the stream is: the last P.V MFMAs of tile t - 1 (operands kept
// in registers across the barrier) while the first score operands are read,
// S(t + 1) interleaved with the first P.V MFMAs of tile t, then the rest of
// P.V(t) interleaved with the softmax of tile t + 1 (its scores are complete
// by then), which sends P(t + 1) to the other waves through LDS.  The S^T
// accumulator layout of the 32x32x16 MFMA (lane: head lane % 32, tokens
// 8 (v / 4) + 4 (lane / 32) + v % 4) is the A layout P.V needs for each
// 16-token k-step, with the token order permuted the same way on the value's
// side, so P needs no shuffle.
//
// LDS: four 36 KB tile buffers (tiles t (P.V), t + 1 (scores), t + 2 and
// t + 3 in flight) and two 8 KB buffers of P: 160 KB, all of it.  A wave's
// vote (a score far above its head's reference, or a head without one)
// therefore rides on P itself: probabilities are never negative, so the wave
// sets the sign bit of lane 0's first value in its k-step-1 fragment, and
// every wave reads that value back with the fragments.  A pass that saw a
// vote is followed by a pass of scores alone (every head's maximum over the
// split) and a second attention pass with those maxima as references.
//
// The splits of one (sequence, head block) are placed on one XCD so that its
// L2 serves their shared query rows (the grid has the sequence index
// fastest).
constexpr int kT2 = 32;                       // tokens per tile
constexpr int kT2Bytes = kT2 * kRowBytes;     // 36864
constexpr int kT2Buffers = 4;
constexpr int kSparseTiles = kMlaSparseTile32Tokens / kT2;  // tiles of a sparse split on this kernel
static_assert(kSparseTiles == 8, "one row register per wave: 8 tiles x 8 rows = 64 lanes");
constexpr int kT2Copies = kT2 * kChunks / 64 / 4;  // 9 wave copies per wave and tile
constexpr int kP2Bytes = 2 * 4 * 64 * 16;     // P of one tile: 2 k-steps x 4 head groups x 64 lanes x 16 B
static_assert(kT2Buffers * kT2Bytes + 2 * kP2Bytes <= 160 * 1024, "fits the LDS");

// Chunk permutation for the 32-row tiles, measured conflict-free (rocprofv3
// SQ_LDS_BANK_CONFLICT = 0 on gfx950) for both read patterns of this kernel:
// score reads (lane l: row l % 32, chunk 2 k + l / 32, 16 bytes) and
// transpose reads (rows 16 ks + 4 (l / 32) + (l % 16) / 4 and + 8).
__device__ __forceinline__ int swz32(int r) {
  const int m = (r >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}

// Balanced splits: this workgroup's item, its sequence b and token range
// [f_begin, f_begin + n_tok) of the sequence's N tokens, and where its
// partials go (rows pbase + h * pstride: a sequence's items own a block of
// n_b * H rows, head-major, so the combine reads each head's partials in one
// run).  The chunk is the smallest multiple of 32 tokens, within [flat_min,
// flat_max], that cuts the sequences into at most flat_target items (one
// round of workgroups; item counts round up per sequence, so T / target
// alone can overshoot by up to B).  Grid slots reach the 8 XCDs round-robin;
// with n items, slot k holds item (k % 8) * ceil(n / 8) + k / 8, so each XCD
// runs ceil(n / 8) consecutive items, mostly of a few sequences whose query
// rows its L2 then serves.  Every wave plans alike from all B lengths (8 per
// lane); wave 0 of slot 0 writes the item table.

// the chunk for total tokens `tot`, given the item count of a chunk
template <typename F>
__device__ __forceinline__ int flat_chunk(const MlaArgs& a, int64_t tot, const F& items_of, int& items) {
  int chunk = (int)max((tot + a.flat_target - 1) / a.flat_target, (int64_t)a.flat_min);
  chunk = min((chunk + kT2 - 1) / kT2 * kT2, a.flat_max);
  items = items_of(chunk);
  for (int it = 0; it < 8 && items > a.flat_target && chunk < a.flat_max; ++it) {
    // grow by the share of items over the target (at least a tile)
    const int grow = max(kT2, (int)((int64_t)chunk * (items - a.flat_target) / a.flat_target));
    chunk = min((chunk + grow + kT2 - 1) / kT2 * kT2, a.flat_max);
    items = items_of(chunk);
  }
  return chunk;
}

// The sequence this slot's item belongs to if every sequence held `cap`
// tokens (scalar; no loads), or -1: a guess to load query rows early.
__device__ __forceinline__ int flat_guess(const MlaArgs& a, int cap) {
  int items, per = 1;
  (void)flat_chunk(a, (int64_t)a.B * cap, [&](int c) { per = (cap + c - 1) / c; return a.B * per; }, items);
  const int k = blockIdx.x, run = (items + 7) >> 3;
  const int item = (k & 7) * run + (k >> 3);
  return (k >> 3) < run && item < items && per > 0 ? item / per : -1;
}

__device__ __forceinline__ void flat_lengths(const MlaArgs& a, int cap, int (&L)[8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int bb = 64 * u + lane;
    L[u] = bb < a.B ? min(max(a.seq_lens[bb], 0), cap) : 0;
  }
}

__device__ __forceinline__ bool flat_place(const MlaArgs& a, const int (&L)[8], bool write_table, int& b, int& N,
                                           int& f_begin, int& n_tok, size_t& pbase, size_t& pstride) {
  const int lane = threadIdx.x & 63;
  int tot = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) tot += L[u];
  tot = __builtin_amdgcn_readfirstlane(__ockl_wfred_add_i32(tot));
  int n[8];
  auto items_of = [&](int c) {
    int s = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      n[u] = 64 * u < a.B ? (L[u] + c - 1) / c : 0;
      s += n[u];
    }
    return __builtin_amdgcn_readfirstlane(__ockl_wfred_add_i32(s));
  };
  int items;
  const int chunk = flat_chunk(a, tot, items_of, items);
  const int k = blockIdx.x, run = (items + 7) >> 3;
  const int item = (k & 7) * run + (k >> 3);
  const bool live = (k >> 3) < run && item < items;
  int running = 0, fb = -1, fj = 0, fl = 0, fo = 0, fn = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (64 * u >= a.B) break;
    int inc = n[u];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d);
      if (lane >= d) inc += y;
    }
    const int excl = running + inc - n[u];
    if (write_table && 64 * u + lane < a.B) {
      a.flat_table[2 * (64 * u + lane)] = excl;
      a.flat_table[2 * (64 * u + lane) + 1] = n[u];
    }
    const uint64_t m = __ballot(live && item >= excl && item < excl + n[u]);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      fb = 64 * u + src;
      fo = __builtin_amdgcn_readlane(excl, src);
      fn = __builtin_amdgcn_readlane(n[u], src);
      fj = item - fo;
      fl = __builtin_amdgcn_readlane(L[u], src);
    }
    running += __builtin_amdgcn_readlane(inc, 63);
  }
  if (fb < 0) return false;
  b = fb;
  N = fl;
  f_begin = fj * chunk;
  n_tok = min(chunk, N - f_begin);
  pbase = (size_t)fo * a.H + fj;
  pstride = (size_t)fn;
  return true;
}

// Where a tile's rows come from: a contiguous cache, a sparse list, or a
// paged cache with pages of at least 8 rows.
enum : int { kSrcContig = 0, kSrcSparse = 1, kSrcPaged = 2 };

// FLAT: balanced items (flat_place) instead of the (B, splits) grid; a
// template parameter, so that the split-grid instances keep their own code.
template <int SRC, bool FLAT = false>
__global__ __launch_bounds__(256, 1) void mla_tile32_kernel(const MlaArgs a) {
  constexpr bool SPARSE = SRC == kSrcSparse;
  constexpr bool PAGED = SRC == kSrcPaged;
  constexpr int kKS = kDq / 16;          // 36 score k-steps of 16 dims
  constexpr int kNT = kDc / 4 / 32;      // 4 output tiles of 32 dims per wave
  constexpr int kP1 = 4;                 // P.V MFMAs in the score phase (of 32)
  constexpr int kDefer = 4;              // P.V MFMAs run after the barrier (of 32)
  static_assert(kDefer % 4 == 0 && kDefer <= 8, "whole head-group rounds, two value fragments");
  const float NEG_INF = -__builtin_inff();
  __shared__ __attribute__((aligned(16))) char tiles[kT2Buffers * kT2Bytes];
  __shared__ __attribute__((aligned(16))) char pbuf[2][kP2Bytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, lj = lane & 31, li = lane & 15, g = lane >> 4;
  const int hw = blockIdx.z * 128;       // the workgroup's first head
  const int h0 = hw + wave * 32;         // this wave's score heads
  const int d0 = wave * 128;             // this wave's output dims

  // the split: positions [f_begin, f_begin + n_tok) of the sequence (or
  // list); its partials go to rows pbase + h * pstride.  Grid (B, splits,
  // H / 128): workgroups reach the 8 XCDs round-robin by linear id, so with
  // the sequence fastest the splits of one sequence share an XCD (B a
  // multiple of 8), and its L2 serves their common query rows.  Balanced
  // splits: grid (slots, 1, H / 128), placed by flat_place.
  constexpr bool flat = FLAT;
  static_assert(!FLAT || SRC == kSrcContig, "paged caches and sparse lists keep the split grid");
  int b = blockIdx.x, split = blockIdx.y;
  int N = 0, f_begin = 0, n_tok = 0;
  size_t pbase = (size_t)b * a.H * a.num_splits + split, pstride = (size_t)a.num_splits;
  // Q^T fragments (B of the scores): lane holds head h0 + lj, dims 16 k + 8 half + [0, 8)
  bf16x8_t qf[kKS];
  int bq = -1;  // the sequence whose query rows qf holds
  auto load_q = [&](int bs) {
    const uint16_t* qrow = a.q + ((size_t)bs * a.H + h0 + lj) * kDq + 8 * half;
#pragma unroll
    for (int k = 0; k < kKS; ++k) qf[k] = *(const bf16x8_t*)(qrow + 16 * k);
    bq = bs;
  };
  if constexpr (flat) {
    // the lengths first, then the query rows of the full-length guess while
    // they are in flight (right for full-length batches; reloaded otherwise)
    const int cap = PAGED ? a.page_size * a.max_pages : a.S_max;
    int L8[8];
    flat_lengths(a, cap, L8);
    const int guess = flat_guess(a, cap);
    if (guess >= 0) load_q(guess);
    if (!flat_place(a, L8, blockIdx.x == 0 && blockIdx.z == 0 && wave == 0, b, N, f_begin, n_tok, pbase,
                    pstride))
      return;
  }
  auto place_split = [&](int len) {
    N = SPARSE ? len : max(0, min(len, PAGED ? a.page_size * a.max_pages : a.S_max));
    const int per = ((N + a.num_splits - 1) / a.num_splits + kT2 - 1) / kT2 * kT2;
    f_begin = min(N, split * per);
    n_tok = min(N, f_begin + per) - f_begin;
  };
  // SPARSE: the split's list entries first (see below); dense: the sequence
  // length; then the query rows while either is in flight
  int len_raw = 0, cids = 0, lid[4] = {-1, -1, -1, -1};
  // PAGED: the page-table entries of the split's pages (at most 128), lane l
  // of pe[0] / pe[1] holding page first_page + l / + 64 + l; requested before
  // the query rows, after the sequence length they depend on
  int pe[2] = {0, 0}, first_page = 0;
  if constexpr (PAGED) {
    if (!flat) place_split(a.seq_lens[b]);
    first_page = f_begin >> a.log2_page;
    const int n_pages = n_tok > 0 ? ((f_begin + n_tok - 1) >> a.log2_page) - first_page + 1 : 0;
    const int32_t* row = a.page_table + (size_t)b * a.max_pages + first_page;
#pragma unroll
    for (int u = 0; u < 2; ++u) pe[u] = 64 * u + lane < n_pages ? row[64 * u + lane] : 0;
  } else if constexpr (SPARSE) {
    place_split(a.k_sel);
    const int32_t* list = a.idx + (size_t)b * a.k_sel + f_begin;
    const int p = 32 * (lane >> 3) + 8 * wave + (lane & 7);
    cids = p < n_tok ? list[p] : -1;
#pragma unroll
    for (int u = 0; u < 4; ++u) lid[u] = 64 * u + lane < n_tok ? list[64 * u + lane] : -1;
  } else {
    if (!flat) len_raw = a.seq_lens[b];
  }
  if (bq != b) load_q(b);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SRC == kSrcContig) {
    if (!flat) place_split(len_raw);
  }
  const int n_tiles = (n_tok + kT2 - 1) / kT2;

  const uint32_t tiles_base = lds_address(tiles);
  const uint32_t pbuf_base = lds_address(pbuf);
  // this lane's slot in a P buffer: reads and writes add uniform offsets
  const uint32_t p_lane = pbuf_base + 16u * (uint32_t)lane;
  auto buffer = [&](int tix) -> uint32_t { return tiles_base + (uint32_t)(tix & 3) * kT2Bytes; };

  // SPARSE (a split of at most kSparseTiles tiles): the validity of each
  // position of the split as a bitmap in scalar registers, and in one
  // register per wave the cache rows its copies need: lane l holds position
  // 32 (l / 8) + 8 wave + l % 8, i.e. row 8 wave + l % 8 of tile l / 8 (a
  // wave's copies cover its rows 8 wave .. 8 wave + 7).  A position without
  // a valid row is masked like a position past the split end and copies the
  // split's first valid row instead (finite data whose P is 0), so every copy
  // instruction is issued whole and the barriers' counts of copies in flight
  // stay exact.
  auto valid_row = [&](int id) -> bool { return id >= 0 && id < a.S_max; };
  // (the list entries were requested before the query rows, so waiting for
  // them here leaves the query rows in flight)
  uint64_t vb0 = 0, vb1 = 0, vb2 = 0, vb3 = 0;  // positions 0-63, .., 192-255
  int fill = 0;
  int n_tiles_run = n_tiles;
  if constexpr (SPARSE) {
    const int32_t* list = a.idx + (size_t)b * a.k_sel + f_begin;
    vb0 = __ballot(valid_row(lid[0]));
    vb1 = __ballot(valid_row(lid[1]));
    vb2 = __ballot(valid_row(lid[2]));
    vb3 = __ballot(valid_row(lid[3]));
    const int first = vb0 ? __builtin_ctzll(vb0)
                    : vb1 ? 64 + __builtin_ctzll(vb1)
                    : vb2 ? 128 + __builtin_ctzll(vb2)
                    : vb3 ? 192 + __builtin_ctzll(vb3) : -1;
    if (first < 0) n_tiles_run = 0;  // no valid row: nothing to attend
    else fill = list[first];
  }
  // SPARSE: positions of tile tix without a valid row (bit r: position r)
  auto holes_of = [&](int tix) -> uint32_t {
    if (tix >= kSparseTiles) return ~0u;
    const uint64_t w = tix < 2 ? vb0 : tix < 4 ? vb1 : tix < 6 ? vb2 : vb3;
    return ~(uint32_t)(w >> (32 * (tix & 1)));
  };

  // ---- copies: wave copy j fills slots 576 wave + 64 j + lane of a tile;
  // slot q is row q / 72, stored chunk q % 72, logical chunk (q % 72) ^ f(row).
  // Byte offset within the tile of this lane's source for each copy, for
  // whole tiles; the last tile clamps rows past the split end to its last.
  uint32_t coff2[(kT2Copies + 1) / 2];  // two 16-bit offsets per register
#pragma unroll
  for (int j = 0; j < kT2Copies; ++j) {
    const uint32_t q = (uint32_t)(576 * wave + 64 * j + lane);
    const uint32_t r = q / kChunks, cs = q - r * kChunks;
    const uint32_t c = (cs & ~7u) | ((cs & 7u) ^ (uint32_t)swz32((int)r));
    const uint32_t off = r * kRowBytes + c * 16;  // < 2^16
    if (j % 2 == 0) coff2[j / 2] = off;
    else coff2[j / 2] |= off << 16;
  }
  auto coff = [&](int j) -> uint32_t { return j % 2 == 0 ? coff2[j / 2] & 0xffffu : coff2[j / 2] >> 16; };
  const char* latent = (const char*)a.latent + (SRC == kSrcContig ? ((size_t)b * a.S_max + f_begin) * kRowBytes
                                                : SPARSE ? (size_t)b * a.S_max * kRowBytes : 0);
  auto tile_src = [&](int tix) -> const char* { return latent + (size_t)tix * kT2Bytes; };
  // source offset of copy j for tile tix (rows past the split end re-read its
  // last row: finite data whose P is 0)
  auto copy_off = [&](int tix, int j, bool whole) -> uint32_t {
    const uint32_t o = coff(j);
    if (whole) return o;
    const int rows_here = n_tok - tix * kT2;
    const uint32_t r = o / kRowBytes;
    return min(r, (uint32_t)(max(rows_here, 1) - 1)) * kRowBytes + (o - r * kRowBytes);
  };
  // whole: the tile holds kT2 tokens of the split (no clamping)
  auto copy = [&](int tix, int j, bool whole) {
    const uint32_t dst = buffer(tix) + 16u * (uint32_t)(576 * wave) + 1024u * j;
    if constexpr (SPARSE) {
      // copy j covers slots 64 j .. 64 j + 63 of the wave's eight rows:
      // row lo, and row lo + 1 from lane thr on
      const int lo = 64 * j / kChunks, thr = kChunks * (lo + 1) - 64 * j;
      const int r_lo = __builtin_amdgcn_readlane(cids, 8 * tix + lo);
      const int r_hi = thr < 64 ? __builtin_amdgcn_readlane(cids, 8 * tix + lo + 1) : r_lo;
      const bool up = lane >= thr;
      const int rid = up ? r_hi : r_lo;
      const uint32_t c16 = coff(j) - (uint32_t)(8 * wave + lo + (up ? 1 : 0)) * kRowBytes;
      copy_to_lds_sv((uint32_t)(valid_row(rid) ? rid : fill) * kRowBytes + c16, latent, dst);
    } else if constexpr (PAGED) {
      // the wave's eight rows of the tile lie in one page (pages of >= 8
      // rows, tiles at multiples of 32); rows past the split end re-read its
      // last row, in the last row's page when the whole block is past it
      const int p0 = min(tix * kT2 + 8 * wave, n_tok - 1);  // the block's first row, in the split
      const int pos = f_begin + p0;
      const int pg = (pos >> a.log2_page) - first_page;
      const int phys = __builtin_amdgcn_readlane(pg < 64 ? pe[0] : pe[1], pg & 63);
      const int64_t row0 = (int64_t)phys * a.page_size + (pos & (a.page_size - 1));
      if (whole) {
        copy_to_lds_sv(coff(j), latent + (row0 - 8 * wave) * kRowBytes, dst);
      } else {
        const uint32_t o = coff(j);
        const uint32_t r = o / kRowBytes;  // tile row 8 wave + i
        const uint32_t i = min(r - 8u * (uint32_t)wave, (uint32_t)(n_tok - 1 - p0));
        copy_to_lds_sv(i * kRowBytes + (o - r * kRowBytes), latent + row0 * kRowBytes, dst);
      }
    } else {
      copy_to_lds_sv(copy_off(tix, j, whole), tile_src(tix), dst);
    }
  };
  auto issue = [&](int tix) {
#pragma unroll
    for (int j = 0; j < kT2Copies; ++j) copy(tix, j, false);
  };

  // ---- per-lane parts of the LDS reads
  const int sw_a = swz32(lj);                 // scores: row lj, chunk 2 k + half
  const int rv = 4 * half + (li >> 2);         // values: rows 16 ks + rv and + 8
  const int cv = 2 * (g & 1) + ((li >> 1) & 1);  // chunk 16 wave + 4 nt + cv, byte 8 (li & 1)
  const int sw_v0 = swz32(rv), sw_v1 = swz32(rv + 8);  // the same for every ks (rows + 16)

  f32x16_t acc[16];  // [hg * kNT + nt]: heads hw + 32 hg + .., dims d0 + 32 nt + ..
  auto zero_acc = [&]() {
    const bf16x8_t z = {};
#pragma unroll
    for (int n = 0; n < 16; ++n)
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc[n]) : "v"(z));
  };
  zero_acc();
  // head h0 + lj: reference maximum (log2 units), largest score seen, this
  // lane's share of the denominator
  float m_run = NEG_INF, m_seen = NEG_INF, l_run = 0.f;

  // Softmax of one tile's scores s (tile tix) in steps of a few VALU
  // instructions, one per P.V MFMA (a matrix-core instruction hides a
  // handful).  Three kinds of pass use it:
  //   full (kXSteps steps, the first tile of a pass): each head's maximum over
  //     the tile becomes its reference unless it has one; a head left without
  //     one (no score in the tile) votes;
  //   lean (kXLean, every later tile): no maximum; a lane votes when its 16
  //     probabilities sum past 2^kTau, which any score past the reference by
  //     more than kTau makes them do;
  //   max (kXMax): only each head's maximum, into m_seen.
  // Full and lean write the tile's P, and the wave's vote in its k-step 1
  // fragment, to pbuf[tix & 1].
  constexpr int kFull = 0, kLean = 1, kMaxOnly = 2;
  constexpr int kXSteps = 16, kXLean = 11, kXMax = 4;
  float m8a, m8b, mxs, mx, nmu, tsum;
  uint4 pv;
  bool jump = false;
  auto exp_pair = [&](f32x16_t& s, int v0) {
    s[v0] = fast_exp2(__builtin_fmaf(s[v0], a.scale_log2, nmu));
    s[v0 + 1] = fast_exp2(__builtin_fmaf(s[v0 + 1], a.scale_log2, nmu));
  };
  // P of k-step ks: tokens 16 ks + 8 (v / 4) + 4 half + v % 4 for v = 8 ks ..
  // 8 ks + 7, in the 32x32x16 A layout; k-step 1 carries the vote on the sign
  // bit of lane 0's first value
  auto pack = [&](const f32x16_t& s, int ks) {
    pv.x = pack_bf16x2(s[8 * ks + 0], s[8 * ks + 1]);
    pv.y = pack_bf16x2(s[8 * ks + 2], s[8 * ks + 3]);
    pv.z = pack_bf16x2(s[8 * ks + 4], s[8 * ks + 5]);
    pv.w = pack_bf16x2(s[8 * ks + 6], s[8 * ks + 7]);
    if (ks == 1) {
      const bool any = __ballot(jump) != 0;
      if (lane == 0) pv.x = (pv.x & 0xffff7fffu) | (any ? 0x8000u : 0u);
    }
  };
  auto put = [&](int tix, int ks) {
    const uint32_t dst = p_lane + (uint32_t)(tix & 1) * kP2Bytes + 1024u * (uint32_t)(ks * 4 + wave);
    *(lds_bf16x8*)(uintptr_t)dst = __builtin_bit_cast(bf16x8_t, pv);
  };
  auto xpiece = [&](auto mode, f32x16_t& s, int tix, int k) {
    constexpr int MODE = decltype(mode)::value;
    if (k == 0) {
      if constexpr (SPARSE) {
        const uint32_t holes = holes_of(tix);
        if (holes != 0u) {
          const uint32_t hl = holes >> (4 * half);  // bit 8 (v / 4) + v % 4: token of s[v]
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if ((hl >> (8 * (v / 4) + (v % 4))) & 1u) s[v] = NEG_INF;
        }
      } else if (__builtin_amdgcn_readfirstlane(tix * kT2 + kT2 > n_tok)) {  // positions past the split end
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (tix * kT2 + 8 * (v / 4) + 4 * half + (v % 4) >= n_tok) s[v] = NEG_INF;
      }
    }
    if constexpr (MODE == kLean) {
      // 1..8: exponentials of s[0..15] (k-step 0's P packed at 5, stored at
      // 6); 9: the sum, the vote, k-step 1's P; 10: stored
      if (k >= 1 && k <= 8) {
        const int v0 = 2 * (k - 1);
        exp_pair(s, v0);
        const float two = s[v0] + s[v0 + 1];
        tsum = k == 1 ? two : tsum + two;
      }
      if (k == 5) pack(s, 0);
      if (k == 6) put(tix, 0);
      if (k == 9) {
        jump = tsum > kTwoTau;
        l_run += tsum;
        pack(s, 1);
      }
      if (k == 10) put(tix, 1);
    } else {
      if (k == 0) {
        m8a = max3(s[0], s[1], max3(s[2], s[3], s[4]));
      } else if (k == 1) {
        m8b = max3(s[5], s[6], max3(s[7], s[8], s[9]));
      } else if (k == 2) {
        const float m8c = max3(s[10], s[11], max3(s[12], s[13], max2(s[14], s[15])));
        mxs = max3(m8a, m8b, m8c);
      } else if (k == 3) {
        // lanes lj and lj + 32 hold the two halves of head lj's tokens
        const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(mxs), __float_as_uint(mxs), false, false);
        mx = max2(__uint_as_float(w[0]), __uint_as_float(w[1])) * a.scale_log2;
        if constexpr (MODE == kMaxOnly) m_seen = max2(m_seen, mx);
      } else if constexpr (MODE == kFull) {
        if (k == 4) {
          m_run = m_run == NEG_INF ? mx : m_run;
          jump = m_run == NEG_INF;
          nmu = m_run == NEG_INF ? 0.f : -m_run;
        } else if ((k >= 5 && k < 9) || (k >= 10 && k < 14)) {
          const int v0 = 2 * (k < 9 ? k - 5 : k - 6);
          exp_pair(s, v0);
          l_run += s[v0] + s[v0 + 1];
        } else if (k == 9) {
          pack(s, 0);
        } else if (k == 14) {
          pack(s, 1);
        }
        if (k == 10) put(tix, 0);
        if (k == 15) put(tix, 1);
      }
    }
  };

  // Scores of the tile in buffer sbuf (36 MFMAs), optionally interleaved with
  // P.V MFMAs, copies and softmax pieces via the hook called at each k-step.
  // this lane's parts of the operand addresses within a tile buffer, kept in
  // registers except by the paged kernel (whose page entries take their place)
  auto so_part = [&](int j) -> uint32_t { return lj * kRowBytes + 16 * ((2 * j + half) ^ sw_a); };
  auto vo_part = [&](int j) -> uint32_t {
    return (j < 2 ? rv : rv + 8) * kRowBytes + 16 * (16 * wave + ((4 * (j & 1) + cv) ^ (j < 2 ? sw_v0 : sw_v1))) +
           8 * (li & 1);
  };
  uint32_t so_lane[4], vo_lane[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    so_lane[j] = PAGED ? 0u : so_part(j);
    vo_lane[j] = PAGED ? 0u : vo_part(j);
  }
  auto a_addr = [&](uint32_t sbuf, int j) -> uint32_t {  // chunk 2 k + half = 8 (k / 4) + (2 (k % 4) + half)
    return sbuf + (PAGED ? so_part(j) : so_lane[j]);
  };

  // P.V MFMA u (0..31): k-step u / 16, output tile (u / 4) % 4, head group u % 4
  auto pv_mfma = [&](int u, const bf16x8_t (&pa)[4], const bf16x8_t (&vr)[2]) {
    const int nt = (u >> 2) & 3, hg = u & 3;
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(acc[hg * kNT + nt]) : "v"(pa[hg]), "v"(vr[nt & 1]));
  };

  // P fragments of one k-step (head groups) and value fragments; the last
  // kDefer P.V MFMAs of a tile keep theirs across the barrier
  bf16x8_t pa[4], vr[2];
  auto defer_mfma = [&](int i) { pv_mfma(32 - kDefer + i, pa, vr); };

  // The stream of iteration t: S(t + 1) || P.V(t) || softmax(t + 1) || copies of
  // t + 3: none (kCopy = 0), of a whole tile (1) or of the split's last,
  // partial tile (2).  It opens with the last kDefer P.V MFMAs of tile t - 1,
  // whose operands are in registers, while the first LDS reads are in flight.
  auto stream = [&](auto mode, auto copy_kind, int t, f32x16_t& s, bool& vote) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool PV = MODE != kMaxOnly;  // the max pass has no P.V
    constexpr int kCopy = decltype(copy_kind)::value;
    const uint32_t sbuf = buffer(t + 1), vbuf = buffer(t);
    const uint32_t pin = p_lane + (uint32_t)(t & 1) * kP2Bytes;
    uint32_t so[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      so[j] = a_addr(sbuf, j);
      asm volatile("" : "+v"(so[j]));
    }
    uint32_t vo[4];  // rows rv (+ 8), chunk groups 0 and 1 of the wave's 128 dims
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      vo[j] = vbuf + (PAGED ? vo_part(j) : vo_lane[j]);
      vo[2 + j] = vbuf + (PAGED ? vo_part(2 + j) : vo_lane[2 + j]);
      asm volatile("" : "+v"(vo[j]), "+v"(vo[2 + j]));
    }
    auto aread = [&](int k) -> bf16x8_t {
      return *(const lds_bf16x8*)(uintptr_t)(so[k & 3] + 128 * (k >> 2));
    };
    // value fragment of k-step ks, output tile nt: chunk 16 wave + 4 nt + cv
    // = 8 (2 wave + nt / 2) + (4 (nt % 2) + cv), rows + 16 ks
    auto vread = [&](int ks, int nt) -> bf16x8_t {
      const uint32_t imm = 128 * (nt >> 1) + 16 * kRowBytes * ks;
      const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(vo[nt & 1] + imm));
      const bf16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(vo[2 + (nt & 1)] + imm));
      return __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto pread = [&](int ks, int hg) -> bf16x8_t {
      return *(const lds_bf16x8*)(uintptr_t)(pin + 1024u * (uint32_t)(ks * 4 + hg));
    };
    // value fragments: (ks, nt) for MFMAs 16 ks + 4 nt .. + 3, two in flight
    auto vload = [&](int u) {  // load the fragment MFMA u first needs
      const int ks = u >> 4, nt = (u >> 2) & 3;
      vr[nt & 1] = vread(ks, nt);
    };

    // the first score operands first: every wave's first MFMA waits on them
    bf16x8_t ar[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) ar[j] = aread(j);
    __builtin_amdgcn_sched_barrier(0);
    // each head group's P fragment is replaced once its last deferred use is issued
    if constexpr (PV) {
#pragma unroll
      for (int i = 0; i < kDefer; ++i) {
        defer_mfma(i);
        if (i >= kDefer - 4) pa[i % 4] = pread(0, i % 4);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int hg = kDefer; hg < 4; ++hg) pa[hg] = pread(0, hg);
      vload(0);
      vload(4);
    }
    __builtin_amdgcn_sched_barrier(0);

    // phase 1: the 36 score MFMAs, with P.V MFMAs 0 .. kP1 - 1 (at k = 3, 7,
    // 11, 15) and the copies of tile t + 3 early, one after each of k = 1 .. 9
    // (their lead over the barrier that waits for them is then longest)
#pragma unroll
    for (int k = 0; k < kKS; ++k) {
      if (k == 0) asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(ar[0]), "v"(qf[0]));
      else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(ar[k % kRing]), "v"(qf[k]));
      if (k + kRing < kKS) ar[k % kRing] = aread(k + kRing);
      if (PV && k % 4 == 3 && k / 4 < kP1) {
        const int u = k / 4;
        pv_mfma(u, pa, vr);
        if ((u & 3) == 3 && u + 5 < 32) vload(u + 5);
      }
      if constexpr (kCopy > 0) {
        if (k >= 1 && k <= kT2Copies) copy(t + 3, k - 1, kCopy == 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase 2: the P.V MFMAs up to the deferred ones, with the softmax of
    // tile t + 1 between them (its first read of the scores comes two MFMAs
    // after the last score MFMA, past the 18 wait states a 32x32 MFMA result
    // needs)
#pragma unroll
    for (int u = kP1; u < 32 - kDefer; ++u) {
      const int w = u - kP1;
      if constexpr (PV) {
        pv_mfma(u, pa, vr);
        if ((u & 3) == 3 && u + 5 < 32) vload(u + 5);
        // k-step 1's P fragment of a head group once k-step 0's last use is past
        if (u >= 12 && u < 16) pa[u - 12] = pread(1, u - 12);
        // the vote in tile t's P: any wave's sign bit on lane 0's first value
        // of k-step 1 (read once those fragments are in)
        if (u == 20) {
          const uint32_t vote_bits = __builtin_bit_cast(uint4, pa[0]).x | __builtin_bit_cast(uint4, pa[1]).x |
                                     __builtin_bit_cast(uint4, pa[2]).x | __builtin_bit_cast(uint4, pa[3]).x;
          vote = (__builtin_amdgcn_readfirstlane(vote_bits) & 0x8000u) != 0;
        }
      }
      // the softmax of tile t + 1: a max step after each MFMA from the third
      // on; a lean step after every other one, so that its VALU spreads over
      // the whole phase (1.2-1.3 % faster than one after each)
      constexpr int kXStride = MODE == kLean ? 2 : 1;
      constexpr int kXN = MODE == kLean ? kXLean : kXMax;
      static_assert(2 + kXStride * (kXN - 1) < 32 - kP1 - kDefer, "the softmax fits the phase");
      if (w >= 2 && (w - 2) % kXStride == 0 && (w - 2) / kXStride < kXN) xpiece(mode, s, t + 1, (w - 2) / kXStride);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: tiles 0..2 requested; tile 0 scored, its softmax taken and its
  // P in pbuf[0] (the max pass: its maximum taken); tile 1 complete.
  auto prime = [&](auto mode, f32x16_t& s) {
    constexpr int MODE = decltype(mode)::value;
    const int first = min(n_tiles, 3);
    for (int t = 0; t < first; ++t) issue(t);
    if (first == 3) barrier_in_flight<2 * kT2Copies>();
    else if (first == 2) barrier_in_flight<kT2Copies>();
    else barrier_in_flight<0>();
    uint32_t so[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      so[j] = a_addr(buffer(0), j);
      asm volatile("" : "+v"(so[j]));
    }
    bf16x8_t ar[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) ar[j] = *(const lds_bf16x8*)(uintptr_t)(so[j & 3] + 128 * (j >> 2));
#pragma unroll
    for (int k = 0; k < kKS; ++k) {
      if (k == 0) asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(ar[0]), "v"(qf[0]));
      else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(ar[k % kRing]), "v"(qf[k]));
      if (k + kRing < kKS) ar[k % kRing] = *(const lds_bf16x8*)(uintptr_t)(so[(k + kRing) & 3] + 128 * ((k + kRing) >> 2));
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
#pragma unroll
    for (int k = 0; k < (MODE == kFull ? kXSteps : kXMax); ++k) xpiece(mode, s, 0, k);
    if (first >= 3) barrier_in_flight<kT2Copies>();  // tile 1 complete; P(0) visible
    else barrier_in_flight<0>();
  };

  // A pass runs every tile of the split.  The tile loops have no early exit,
  // so the accumulators follow one path.
  f32x16_t s;
  bool vote = false;
  auto tiles_after_first = [&](auto mode) -> bool {
    bool again = false;
    // iterations that request a whole tile, the one that requests the
    // split's partial last tile, then the tail
    const int n_copying = max(n_tiles - 3, 0);
    const int n_whole = min(n_copying, max(n_tok / kT2 - 3, 0));
    int t = 0;
    for (; t < n_whole; ++t) {
      stream(mode, std::integral_constant<int, 1>{}, t, s, vote);
      barrier_in_flight<kT2Copies>();  // tile t + 2 complete, tile t + 3 in flight
      again |= vote;
    }
    for (; t < n_copying; ++t) {
      stream(mode, std::integral_constant<int, 2>{}, t, s, vote);
      barrier_in_flight<kT2Copies>();
      again |= vote;
    }
    for (; t < n_tiles; ++t) {
      stream(mode, std::integral_constant<int, 0>{}, t, s, vote);
      barrier_in_flight<0>();
      again |= vote;
    }
    return again;
  };
  // one pass, each head's reference its first tile's maximum unless set
  auto attention_pass = [&]() -> bool {
    prime(std::integral_constant<int, kFull>{}, s);
    // the first iteration's deferred MFMAs have no tile before them: zero operands
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) pa[hg] = bf16x8_t{};
    vr[0] = vr[1] = bf16x8_t{};
    const bool again = tiles_after_first(std::integral_constant<int, kLean>{});
#pragma unroll
    for (int i = 0; i < kDefer; ++i) defer_mfma(i);
    return again;
  };
  if (n_tiles_run > 0 && attention_pass()) {
    // a vote: some head's score passed its reference by more than kTau, or a
    // head had no score in its first tile.  A pass of scores alone finds
    // every head's maximum over the split; with it as the reference the
    // second attention pass has no jump (a jump needs an ordered comparison,
    // so NaN scores never vote) and its vote is not read.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);  // in-flight MFMAs retire first
    m_seen = NEG_INF;
    prime(std::integral_constant<int, kMaxOnly>{}, s);
    (void)tiles_after_first(std::integral_constant<int, kMaxOnly>{});
    m_run = m_seen;
    zero_acc();
    l_run = 0.f;
    (void)attention_pass();
  }
  settle(acc);

  // unnormalised partials: O (relative to m_run), m_run and l per head
#pragma unroll
  for (int hg = 0; hg < 4; ++hg)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        a.part_o[(pbase + (size_t)(hw + 32 * hg + 8 * (v / 4) + 4 * half + (v % 4)) * pstride) * kDc + d0 +
                 32 * nt + lj] = acc[hg * kNT + nt][v];
  const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(w[0]) + __uint_as_float(w[1]);
  if (half == 0) {
    const size_t r = pbase + (size_t)(h0 + lj) * pstride;
    a.part_lse[r] = l_tot > 0.f ? m_run : NEG_INF;
    a.part_l[r] = l_tot;
  }
}

template <bool SPARSE, bool TABLE, int NW>
hipError_t launch_variant(const MlaArgs& a, hipStream_t s) {
  dim3 grid(a.B, a.num_splits, a.H / (NW * kHeadsPerWave)), block(64 * NW);
  launch_kernel(mla_split_kernel<SPARSE, TABLE, NW>, grid, block, s, a);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_nw(const MlaArgs& a, hipStream_t s) {
  if (a.idx) return launch_variant<true, true, NW>(a, s);
  if (a.page_table) return launch_variant<false, true, NW>(a, s);
  return launch_variant<false, false, NW>(a, s);
}

}  // namespace

int mla_heads_per_workgroup(int H) { return H % 128 == 0 ? 128 : 64; }

bool mla_sparse_on_tile32(const MlaArgs& a) {
  if (!a.idx || a.heads_per_wg != 128 || a.H % 128 != 0 || a.num_splits < 1) return false;
  const int64_t per = ((int64_t)a.k_sel + a.num_splits - 1) / a.num_splits;
  return per <= (int64_t)kSparseTiles * kT2 && (int64_t)a.S_max * kRowBytes < (int64_t(1) << 32);
}

// A paged call runs there when its pages hold at least 8 rows (a power of
// two) and a split spans at most 128 pages.
bool mla_paged_on_tile32(const MlaArgs& a) {
  if (a.idx || !a.page_table || a.heads_per_wg != 128 || a.H % 128 != 0 || a.num_splits < 1) return false;
  if (a.page_size < 8 || (a.page_size & (a.page_size - 1)) != 0) return false;
  const int64_t cap = (int64_t)a.page_size * a.max_pages;
  const int64_t per = ((cap + a.num_splits - 1) / a.num_splits + kT2 - 1) / kT2 * kT2;
  return per / a.page_size + 2 <= 128;
}

bool mla_uses_tile32(const MlaArgs& a) {
  if (a.flat_target > 0) return true;  // the planner took the 32-row kernel's limits
  if (a.num_splits < 1) return false;
  if (!a.idx && !a.page_table && a.heads_per_wg == 128 && a.H % 128 == 0) return true;
  return mla_sparse_on_tile32(a) || mla_paged_on_tile32(a);
}

hipError_t launch_mla(const MlaArgs& a, hipStream_t s) {
  if (mla_uses_tile32(a)) {
    const dim3 grid = a.flat_target > 0 ? dim3(a.flat_slots, 1, a.H / 128) : dim3(a.B, a.num_splits, a.H / 128);
    const bool flat = a.flat_target > 0;
    if (a.idx) launch_kernel(mla_tile32_kernel<kSrcSparse>, grid, dim3(256), s, a);
    else if (a.page_table) launch_kernel(mla_tile32_kernel<kSrcPaged>, grid, dim3(256), s, a);
    else if (flat) launch_kernel(mla_tile32_kernel<kSrcContig, true>, grid, dim3(256), s, a);
    else launch_kernel(mla_tile32_kernel<kSrcContig>, grid, dim3(256), s, a);
    return hipGetLastError();
  }
  if (a.heads_per_wg == 128 && a.H % 128 == 0) return launch_nw<4>(a, s);
  if (a.heads_per_wg == 64 && a.H % 64 == 0) return launch_nw<2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dattn
