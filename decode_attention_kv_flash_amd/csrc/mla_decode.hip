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
// Data movement: the split's cache rows (paged, contiguous or gathered by a
// top-k list) are resolved once into a row table in LDS.  Tiles of 32 rows
// (36 KB) then go from HBM straight into LDS by direct-to-LDS loads
// (global_load_lds_dwordx4: no registers in between) into four tile
// buffers, issued two tiles ahead of use.  Row r of a tile keeps its 16-byte
// chunk c at slot c ^ f(r) within its group of eight chunks; both read
// patterns below are then free of LDS bank conflicts.
//
// Per tile and wave:
//   * S^T[token, head] = C[token, :] . Q^T over 576 dims: 36 32x32x16 bf16
//     MFMAs, A = latent chunks from LDS, B = the wave's 32 query rows held in
//     registers for the whole split;
//   * online softmax in log2 units per head ("All the attentions", section 1:
//     running maximum and sum); the reference maximum is set by the head's
//     first scores and moves only when a score passes it by more than 2^64
//     (exponentials stay finite in fp32 and keep their relative precision);
//     when that happens the workgroup restarts the split with the larger
//     reference, so the 256-value accumulator is never rescaled;
//   * O[head, 0:512] += P . C[:, 0:512]: the S^T accumulator layout is
//     exactly the A operand P needs (heads x tokens, the k order permuted the
//     same way on both operands), and the B operand (tokens x dims) comes
//     from the row-major tile by the gfx950 transpose read ds_read_b64_tr_b16.
// One wave per SIMD cannot hide LDS latency behind other waves, so the loop
// is software-pipelined: iteration t alternates the score MFMAs of tile t + 1
// with the P.V MFMAs of tile t (independent chains), each LDS read issued
// five MFMAs before its use, then runs the softmax of tile t + 1.
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
constexpr int kTile = 32;           // tokens per tile
constexpr int kHeadsPerWave = 32;
constexpr int kTileChunks = kTile * kChunks;              // 2304
constexpr int kTileBytes = kTileChunks * 16;              // 36864
constexpr int kBuffers = 4;
constexpr int kDmaPerTile = kTileChunks / 64;             // 36 wave-wide 1 KB copies
constexpr int kKSteps = kDq / 16;                         // 36 MFMA k-steps for the scores
constexpr int kNTiles = kDc / 32;                         // 16 output tiles of 32 dims
constexpr int kPvSteps = 2 * kNTiles;                     // 2 k-steps of 16 tokens x 16 tiles
constexpr int kRing = 3;                                  // LDS fragments in flight per operand
constexpr float kTau = 64.0f;                             // reference-maximum slack (log2)
constexpr uint32_t kPad = 0x80000000u;                    // row-table flag: no token here
constexpr int kMaxTiles = kMlaMaxSplitTokens / kTile;
// tiles t + 1 (scores) and up to t + 3 (prefetch) of the last iteration
constexpr int kRowTable = (kMaxTiles + 3) * kTile;
static_assert(kMlaMaxSplitTokens % kTile == 0, "splits hold whole tiles");
static_assert(kBuffers * kTileBytes + kRowTable * 4 + 16 <= 160 * 1024, "fits the LDS");

// Chunk permutation of row r (low three bits of the chunk index only).  LDS
// has 64 four-byte banks; a 16-byte read serves 16 lanes per pass and an
// 8-byte read 32.  Rows are 1152 B apart, i.e. alternate between two
// 128-byte halves of the bank space, so rows of equal parity among 16
// consecutive ones must take distinct slots (score reads: 16 rows, one
// chunk), and rows r, r + 2 (r % 4 < 2) must take slots in different halves
// of an 8-chunk group (transpose reads: 4 rows, 4 chunks).  m -> (m & 1) << 2
// | m >> 1 over m = (r / 2) % 8 does both.
__device__ __forceinline__ int swz(int r) {
  const int m = (r >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;

// The O accumulators are written by MFMAs the compiler does not see; before
// ordinary code reads or writes them, let the last of those MFMAs retire
// (more than the 18 wait states a 32x32 MFMA result needs) and make every
// later access depend on this point.
__device__ __forceinline__ void settle(f32x16_t (&acc)[kNTiles]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
#pragma unroll
  for (int n = 0; n < kNTiles; ++n) asm volatile("" : "+a"(acc[n]));
}

template <bool SPARSE, bool PAGED, int NW>
__global__ __launch_bounds__(64 * NW, 1) void mla_split_kernel(const MlaArgs a) {
  constexpr int kThreads = 64 * NW;
  constexpr int kDmaPerWave = kDmaPerTile / NW;
  static_assert(kDmaPerTile % NW == 0, "copies split evenly over the waves");
  const float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(16))) char tiles[kBuffers * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint32_t rows[kRowTable];
  __shared__ int first_valid;
  // bit t: tile t holds a position without a token (its scores need the mask)
  __shared__ uint32_t tile_pad[(kMaxTiles + 3 + 31) / 32];
  // restart votes: iteration u votes in slot u % 3, every wave reads it after
  // the iteration's barrier, and iteration u + 2 clears it, so a fast wave
  // never touches a vote a slow wave has yet to read
  __shared__ int restart_vote[3];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;   // 32-lane half
  const int lj = lane & 31;
  const int split = blockIdx.x;
  const int b = blockIdx.z;
  const int h0 = blockIdx.y * (NW * kHeadsPerWave) + wave * kHeadsPerWave;

  int N;
  if constexpr (SPARSE) {
    N = a.k_sel;
  } else {
    const int cap = PAGED ? a.page_size * a.max_pages : a.S_max;
    N = max(0, min(a.seq_lens[b], cap));
  }
  const int per = ((N + a.num_splits - 1) / a.num_splits + kTile - 1) / kTile * kTile;
  const int f_begin = min(N, split * per);
  const int f_end = min(N, f_begin + per);
  int n_tiles = min((f_end - f_begin + kTile - 1) / kTile, kMaxTiles);

  // Q^T fragments (B operand): lane holds head h0 + lj, dims 16 ks + 8 half + [0, 8)
  bf16x8_t qf[kKSteps];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.H + h0 + lj) * kDq + 8 * half;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *(const bf16x8_t*)(qrow + 16 * ks);
  }

  // ---- row table: cache row of every position of the split and of the
  // three tiles past it.  Flag kPad marks a position without a token; its
  // entry still names a row of finite data (a real row of the same split),
  // so that P = 0 times it stays 0.
  if (threadIdx.x < (kMaxTiles + 3 + 31) / 32) tile_pad[threadIdx.x] = 0u;
  if (threadIdx.x == 0) {
    first_valid = 0x7fffffff;
    restart_vote[0] = restart_vote[1] = restart_vote[2] = 0;
  }
  __syncthreads();
  const int n_rows = n_tiles > 0 ? (n_tiles + 3) * kTile : 0;
  for (int i = threadIdx.x; i < n_rows; i += kThreads) {
    const int f = f_begin + i;
    uint32_t e;
    if constexpr (SPARSE) {
      const int t = f < f_end ? a.idx[(size_t)b * a.k_sel + f] : -1;
      const bool ok = t >= 0 && t < a.S_max;
      e = ok ? (uint32_t)b * (uint32_t)a.S_max + (uint32_t)t : kPad;
      if (ok) atomicMin(&first_valid, i);
    } else {
      const bool ok = f < f_end;
      const int t = ok ? f : f_end - 1;
      uint32_t row;
      if constexpr (PAGED) {
        const int phys = a.page_table[(size_t)b * a.max_pages + (t >> a.log2_page)];
        row = (uint32_t)phys * (uint32_t)a.page_size + (uint32_t)(t & (a.page_size - 1));
      } else {
        row = (uint32_t)b * (uint32_t)a.S_max + (uint32_t)t;
      }
      e = row | (ok ? 0u : kPad);
    }
    rows[i] = e;
    if (e & kPad) atomicOr(&tile_pad[(i / kTile) >> 5], 1u << ((i / kTile) & 31));
  }
  __syncthreads();
  if constexpr (SPARSE) {
    const int fv = first_valid;
    if (fv == 0x7fffffff) {
      n_tiles = 0;  // nothing to attend in this split
    } else {
      const uint32_t fb = rows[fv] | kPad;
      for (int i = threadIdx.x; i < n_rows; i += kThreads)
        if (rows[i] == kPad) rows[i] = fb;
      __syncthreads();
    }
  }

  const uint32_t tiles_base = lds_address(tiles);
  auto buffer = [&](int tix) -> uint32_t {
    return tiles_base + (uint32_t)(tix & (kBuffers - 1)) * kTileBytes;
  };

  // ---- tile copy: wave copy i (of 36) fills slots 64 i + lane; slot q is
  // row q / 72, stored chunk q % 72, i.e. chunk (q % 72) ^ f(row)
  // This lane's slot in each copy: tile row r and stored chunk c' (a wave's
  // copies cover tile rows 32 w / NW .. + 32 / NW - 1).  With 4 waves the
  // nine slots are kept packed, ten bits each (row within the wave's eight,
  // chunk); with 2 waves they are recomputed per tile (no registers spare).
  auto slot_of = [&](uint32_t q) -> uint32_t {  // row | chunk << 8
    const uint32_t r = q / kChunks;
    return r | (((q - r * kChunks) ^ swz(r)) << 8);
  };
  uint32_t slot_pk[3] = {0u, 0u, 0u};
  if constexpr (NW == 4) {
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const uint32_t rc = slot_of(64 * (wave * kDmaPerWave + j) + lane);
      slot_pk[j / 3] |= (((rc & 0xff) - 8 * wave) | ((rc >> 8) << 3)) << (10 * (j % 3));
    }
  }
  auto issue = [&](int tix) {
    const uint32_t dst = buffer(tix) + 1024u * (uint32_t)(wave * kDmaPerWave);
    const uint32_t* rt = rows + tix * kTile;
    constexpr int kBatch = 9;  // row lookups in flight together
    static_assert(kDmaPerWave % kBatch == 0, "whole batches");
    uint32_t pk[3] = {slot_pk[0], slot_pk[1], slot_pk[2]};
    asm volatile("" : "+v"(pk[0]), "+v"(pk[1]), "+v"(pk[2]));  // unpack here, not once per kernel
#pragma unroll
    for (int j0 = 0; j0 < kDmaPerWave; j0 += kBatch) {
      uint32_t rc[kBatch], row[kBatch];  // rc: row | chunk << 8 of this lane's slot
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if constexpr (NW == 4) {
          const uint32_t x = pk[j / 3] >> (10 * (j % 3));
          rc[j] = (8 * wave + (x & 7)) | (((x >> 3) & 127) << 8);
        } else {
          uint32_t q = 64 * (wave * kDmaPerWave + j0 + j) + lane;
          asm volatile("" : "+v"(q));  // recomputed per tile: registers are the scarce resource
          rc[j] = slot_of(q);
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) row[j] = rt[rc[j] & 0xff] & ~kPad;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const uint64_t chunk = (uint64_t)row[j] * kChunks + (rc[j] >> 8);
        copy_to_lds((const char*)a.latent + 16 * chunk, dst + 1024u * (j0 + j));
      }
    }
  };

  // ---- per-lane parts of the two LDS read patterns
  const int sw_lj = swz(lj);
  const int li = lane & 15, g = lane >> 4;
  const int r1 = 4 * half + (li >> 2);                 // token of k elements 0..3 (+16 kk, +8)
  const int c0 = 2 * (g & 1) + ((li >> 1) & 1);        // chunk of dims 32 n + 16 (g&1) + 4 (li&3)
  const int sw_r1 = swz(r1), sw_r9 = swz(r1 + 8);      // rows + 16 share them

  // O accumulators: defined (zeroed) by MFMAs with zero operands, so that
  // they are born in AGPRs and never pass through VGPRs
  f32x16_t acc[kNTiles];
  auto zero_acc = [&]() {
    const bf16x8_t z = {};
#pragma unroll
    for (int n = 0; n < kNTiles; ++n)
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc[n]) : "v"(z));
  };
  zero_acc();
  // m_run: the head's reference maximum (log2 units); m_seen: largest score so far
  float m_run = NEG_INF, m_seen = NEG_INF, l_run = 0.f;
  bf16x8_t pa[2];  // P of the tile whose P.V comes next, bf16, one per 16-token k-step

  // Scores of the tile in buffer sbuf (S^T, 32 tokens x 32 heads: lane holds
  // head lj, tokens 8(v/4) + 4 half + v%4), alternated with the P.V MFMAs of
  // the tile in buffer pbuf when WITH_PV.
  auto scores = [&](auto with_pv, uint32_t sbuf, uint32_t pbuf) -> f32x16_t {
    constexpr bool WITH_PV = decltype(with_pv)::value;
    // Per-lane LDS addresses, made opaque here so that the compiler keeps
    // eight per tile instead of an address per read.
    // A operand of the scores: row lj, chunk c = 2 ks + half, stored at slot
    // 8 (c / 8) + ((c % 8) ^ f(lj)): so[ks % 4] + 128 (ks / 4).
    // B operand of P.V: rows r1 + 16 kk and r1 + 8 + 16 kk, chunk c = 4 n +
    // c0, stored at 8 (c / 8) + ((c % 8) ^ f(row)): vo[n % 2] and
    // vo[2 + n % 2], + 128 (n / 2) + 16 kk rows.
    uint32_t so[4], vo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      so[j] = sbuf + lj * kRowBytes + 16 * (((2 * j) | half) ^ sw_lj);
      asm volatile("" : "+v"(so[j]));
    }
    if constexpr (WITH_PV) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        vo[j] = pbuf + r1 * kRowBytes + 16 * ((4 * j + c0) ^ sw_r1) + 8 * (li & 1);
        vo[2 + j] = pbuf + (r1 + 8) * kRowBytes + 16 * ((4 * j + c0) ^ sw_r9) + 8 * (li & 1);
        asm volatile("" : "+v"(vo[j]), "+v"(vo[2 + j]));
      }
    }
    auto aread = [&](int ks) -> bf16x8_t {
      return *(const lds_bf16x8*)(uintptr_t)(so[ks & 3] + 128 * (ks >> 2));
    };
    auto vread = [&](int p) -> bf16x8_t {  // p = 16 kk + n
      const int kk = p >> 4, n = p & 15;
      const uint32_t imm = 128 * (n >> 1) + 16 * kk * kRowBytes;
      const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(vo[n & 1] + imm));
      const bf16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(vo[2 + (n & 1)] + imm));
      return __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8_t ar[kRing], vr[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      ar[j] = aread(j);
      if constexpr (WITH_PV) vr[j] = vread(j);
    }
    f32x16_t s;
    asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(ar[0]), "v"(qf[0]));
#pragma unroll
    for (int i = 0; i < kKSteps; ++i) {
      if (i > 0)
        asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+v"(s) : "v"(ar[i % kRing]), "v"(qf[i]));
      if (i + kRing < kKSteps) ar[i % kRing] = aread(i + kRing);
      if constexpr (WITH_PV) {
        if (i < kPvSteps) {
          asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                       : "+a"(acc[i & (kNTiles - 1)]) : "v"(pa[i >> 4]), "v"(vr[i % kRing]));
          if (i + kRing < kPvSteps) vr[i % kRing] = vread(i + kRing);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the scores are read by ordinary code next: let the last MFMA retire
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
    return s;
  };

  // Online softmax of tile tix from its scores s; leaves its P in pa and
  // votes for a restart in restart_vote[slot] when a maximum jumps.
  auto softmax = [&](f32x16_t s, int tix, int slot) {
    // maximum over the raw scores (the scale is positive), masking only in
    // tiles that hold positions without a token
    float mx = NEG_INF;
    if ((tile_pad[tix >> 5] >> (tix & 31)) & 1u) {
      const uint32_t* rt = rows + tix * kTile + 4 * half;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint4 e = *(const uint4*)(rt + 8 * q4);
        const uint32_t ev[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int v = 4 * q4 + u;
          if (ev[u] & kPad) s[v] = NEG_INF;
          mx = fmaxf(mx, s[v]);
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
    }
    // lanes lj and lj + 32 hold the two halves of head lj's tokens
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
    }
    m_seen = fmaxf(m_seen, mx);
    // a head's first scores set its reference (its O is still zero); a later
    // score past the reference by more than kTau asks for a restart
    if (m_run != NEG_INF && mx > m_run + kTau) restart_vote[slot] = 1;
    if (m_run == NEG_INF) m_run = mx;
    const float nmu = m_run == NEG_INF ? 0.f : -m_run;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = fast_exp2(__builtin_fmaf(s[v], a.scale_log2, nmu));
      psum += s[v];
    }
    l_run += psum;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 p;
      p.x = pack_bf16x2(s[8 * kk + 0], s[8 * kk + 1]);
      p.y = pack_bf16x2(s[8 * kk + 2], s[8 * kk + 3]);
      p.z = pack_bf16x2(s[8 * kk + 4], s[8 * kk + 5]);
      p.w = pack_bf16x2(s[8 * kk + 6], s[8 * kk + 7]);
      pa[kk] = __builtin_bit_cast(bf16x8_t, p);
    }
  };

  // Prologue: tiles 0..2 requested, tile 0 scored and its softmax taken,
  // tile 1 complete in LDS.  (A prologue never votes: its reference is unset
  // or already the largest score seen.)
  // Tiles past the split are never copied (their positions are all masked,
  // so whatever their buffers hold never reaches a result).
  auto prime = [&]() {
    issue(0);
    if (n_tiles > 1) issue(1);
    if (n_tiles > 2) issue(2);
    if (n_tiles > 2) barrier_in_flight<2 * kDmaPerWave>();  // tile 0 complete
    else if (n_tiles > 1) barrier_in_flight<kDmaPerWave>();
    else barrier_in_flight<0>();
    softmax(scores(std::false_type{}, buffer(0), 0u), 0, 0);
    if (n_tiles > 2) barrier_in_flight<kDmaPerWave>();  // tile 1 complete
    else barrier_in_flight<0>();
  };

  // Iteration t: request tile t + 3 if the split has it (into the buffer
  // tile t - 1 freed), P.V of tile t alternated with the scores of tile t + 1
  // (for the last t a padding tile, all flagged: its softmax changes
  // nothing), then the softmax of tile t + 1.  Once no tile is requested the
  // barrier waits for every copy, so none is in flight when the workgroup
  // ends.  A restart leaves the tile loop and runs the prologue again.
  while (n_tiles > 0) {
    prime();
    int slot = 0;
    bool again = false;
    for (int t = 0; t < n_tiles; ++t) {
      if (threadIdx.x == 0) restart_vote[slot == 2 ? 0 : slot + 1] = 0;  // iteration t - 2's
      const bool more = t + 3 < n_tiles;
      if (more) issue(t + 3);
      const f32x16_t s = scores(std::true_type{}, buffer(t + 1), buffer(t));
      softmax(s, t + 1, slot);
      // tile t + 2 complete in LDS for every wave (only tile t + 3 may still
      // be in flight); buffer of tile t free for reuse
      if (more) barrier_in_flight<kDmaPerWave>();
      else barrier_in_flight<0>();
      if (restart_vote[slot]) {
        again = true;
        break;
      }
      slot = slot == 2 ? 0 : slot + 1;
    }
    if (!again) break;
    // some head's maximum jumped: redo the split with every head's reference
    // at the largest score it has seen (each restart raises a reference by
    // more than kTau, so restarts are few)
    barrier_in_flight<0>();  // every wave has read the vote; no copy in flight
    if (threadIdx.x == 0) restart_vote[0] = restart_vote[1] = restart_vote[2] = 0;
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);  // in-flight MFMAs retire first
    zero_acc();
    m_run = m_seen;
    l_run = 0.f;
  }
  settle(acc);

  // unnormalised partials: O (relative to m_run), m_run and l per head; the
  // combine merges the splits and divides
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const size_t row0 = (size_t)b * a.H + h0;
#pragma unroll
  for (int n = 0; n < kNTiles; ++n)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      a.part_o[((row0 + 8 * (v / 4) + 4 * half + (v % 4)) * a.num_splits + split) * kDc + 32 * n + lj] =
          acc[n][v];
  if (half == 0) {
    a.part_lse[(row0 + lj) * a.num_splits + split] = l_tot > 0.f ? m_run : NEG_INF;
    a.part_l[(row0 + lj) * a.num_splits + split] = l_tot;
  }
}

template <bool SPARSE, bool PAGED, int NW>
hipError_t launch_variant(const MlaArgs& a, hipStream_t s) {
  dim3 grid(a.num_splits, a.H / (NW * kHeadsPerWave), a.B), block(64 * NW);
  launch_kernel(mla_split_kernel<SPARSE, PAGED, NW>, grid, block, s, a);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_nw(const MlaArgs& a, hipStream_t s) {
  if (a.idx) return launch_variant<true, false, NW>(a, s);
  if (a.page_table) return launch_variant<false, true, NW>(a, s);
  return launch_variant<false, false, NW>(a, s);
}

}  // namespace

int mla_heads_per_workgroup(int H) { return H % 128 == 0 ? 128 : 64; }

hipError_t launch_mla(const MlaArgs& a, hipStream_t s) {
  if (a.heads_per_wg == 128 && a.H % 128 == 0) return launch_nw<4>(a, s);
  if (a.heads_per_wg == 64 && a.H % 64 == 0) return launch_nw<2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace dattn
