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
// (global_load_lds_dwordx4: no registers in between), three tile buffers
// deep, so two tiles are in flight while one is computed.  Row r of a tile
// keeps its 16-byte chunk c at slot c ^ f(r); both read patterns below are
// then free of LDS bank conflicts.
//
// Per tile and wave:
//   * S^T[token, head] = C[token, :] . Q^T over 576 dims: 36 32x32x16 bf16
//     MFMAs, A = latent chunks from LDS, B = the wave's 32 query rows held in
//     registers for the whole split;
//   * online softmax in log2 units per head ("All the attentions", section 1:
//     running maximum and sum); the reference maximum is set by the head's
//     first scores and moves only when a score passes it by more than 2^64
//     (exponentials stay finite in fp32 and keep their relative precision),
//     so the 256-value accumulator is almost never rescaled;
//   * O[head, 0:512] += P . C[:, 0:512]: the S^T accumulator layout is
//     exactly the A operand P needs (heads x tokens, the k order permuted the
//     same way on both operands), and the B operand (tokens x dims) comes
//     from the row-major tile by the gfx950 transpose read ds_read_b64_tr_b16.
//     O lives in accumulation registers (AGPRs) for the whole split.  All
//     MFMAs are issued by inline assembly that pins each operand to its
//     register file (O in AGPRs; scores, Q and the tile fragments in VGPRs);
//     each carries the wait states the compiler would otherwise insert
//     (a VALU result feeding an MFMA; an MFMA result read by ordinary code).
// P is rounded to bf16 for the MFMA; everything else accumulates in fp32.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kDc = 512;            // c_KV width (the value)
constexpr int kDq = 576;            // latent row: c_KV + k_pe
constexpr int kChunks = kDq / 8;    // 16-byte chunks per row
constexpr int kTile = 32;           // tokens per tile
constexpr int kHeadsPerWave = 32;
constexpr int kTileChunks = kTile * kChunks;              // 2304
constexpr int kTileBytes = kTileChunks * 16;              // 36864
constexpr int kDmaPerTile = kTileChunks / 64;             // 36 wave-wide 1 KB copies
constexpr int kKSteps = kDq / 16;                         // 36 MFMA k-steps for the scores
constexpr int kNTiles = kDc / 32;                         // 16 output tiles of 32 dims
constexpr float kTau = 64.0f;                             // reference-maximum slack (log2)
constexpr uint32_t kPad = 0x80000000u;                    // row-table flag: no token here
constexpr int kNT = 2;                                    // cache policy: nontemporal

constexpr int kGroup = 3 * kTile;                         // tokens per loop iteration
static_assert(kMlaMaxSplitTokens % kGroup == 0, "splits hold whole groups");
constexpr int kRowTable = kMlaMaxSplitTokens + 2 * kTile; // + the tiles prefetched past the end

// chunk permutation of row r (low three bits of the chunk index only)
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that leaves the newest N direct-to-LDS copies of this
// wave in flight: wait until at most N vector-memory operations are
// outstanding and every LDS access of this wave is done, then s_barrier.
// (A plain __syncthreads would drain all copies: its release fence treats
// them as pending LDS writes.)  The signal fences keep the compiler from
// moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void barrier_in_flight() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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

template <bool SPARSE, bool PAGED, int NW>
__global__ __launch_bounds__(64 * NW, 1) void mla_split_kernel(const MlaArgs a) {
  constexpr int kThreads = 64 * NW;
  constexpr int kDmaPerWave = kDmaPerTile / NW;
  static_assert(kDmaPerTile % NW == 0, "copies split evenly over the waves");
  const float NEG_INF = -__builtin_inff();

  // three tile buffers as distinct objects: the compiler then knows that a
  // read of one does not wait for copies into another
  __shared__ __attribute__((aligned(16))) char tile0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char tile1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char tile2[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint32_t rows[kRowTable];
  __shared__ int first_valid;
  // restart votes of the even and odd loop iterations: a vote is read by
  // every wave after the iteration's last barrier and cleared one iteration
  // later, so a fast wave never overwrites a vote a slow wave has yet to read
  __shared__ int restart_vote[2];

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
  // splits hold whole groups of three tiles, so only a sequence's last split
  // computes padded tiles
  const int per = ((N + a.num_splits - 1) / a.num_splits + kGroup - 1) / kGroup * kGroup;
  const int f_begin = min(N, split * per);
  const int f_end = min(N, f_begin + per);
  int n_tiles = min((f_end - f_begin + kTile - 1) / kTile, kMlaMaxSplitTokens / kTile);
  const int n_groups = (n_tiles + 2) / 3;

  // Q^T fragments (B operand): lane holds head h0 + lj, dims 16 ks + 8 half + [0, 8)
  bf16x8_t qf[kKSteps];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.H + h0 + lj) * kDq + 8 * half;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *(const bf16x8_t*)(qrow + 16 * ks);
  }

  // ---- row table: cache row of every position of the split.  Flag kPad
  // marks a position without a token; its entry still names a row of finite
  // data (a real row of the same split), so that P = 0 times it stays 0.
  if (threadIdx.x == 0) {
    first_valid = 0x7fffffff;
    restart_vote[0] = restart_vote[1] = 0;
  }
  __syncthreads();
  // every tile a group touches, plus the two tiles prefetched past the last
  const int n_rows = n_tiles > 0 ? (3 * n_groups + 2) * kTile : 0;
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

  // ---- direct-to-LDS tile copy: wave copy i (of 36) fills slots 64 i + lane;
  // slot q is row q / 72, stored chunk q % 72, i.e. chunk (q % 72) ^ f(row)
  uint32_t dma_rc[kDmaPerWave];  // row | chunk << 8, fixed for the kernel
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int q = 64 * (wave * kDmaPerWave + j) + lane;
    const int r = q / kChunks;
    dma_rc[j] = (uint32_t)r | ((uint32_t)((q - r * kChunks) ^ swz(r)) << 8);
  }
  auto issue = [&](auto buf_id, int tix) {
    constexpr int BI = decltype(buf_id)::value;
    char* buf = BI == 0 ? tile0 : BI == 1 ? tile1 : tile2;
    const uint32_t* rt = rows + tix * kTile;
    constexpr int kBatch = 9;  // row lookups in flight together
    static_assert(kDmaPerWave % kBatch == 0, "whole batches");
#pragma unroll
    for (int j0 = 0; j0 < kDmaPerWave; j0 += kBatch) {
      uint32_t rc[kBatch], row[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        rc[j] = dma_rc[j0 + j];
        asm volatile("" : "+v"(rc[j]));  // keep per-copy addresses out of long-lived registers
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) row[j] = rt[rc[j] & 0xff] & ~kPad;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const uint64_t chunk = (uint64_t)row[j] * kChunks + (rc[j] >> 8);
        __builtin_amdgcn_global_load_lds((const void*)((const char*)a.latent + 16 * chunk),
                                         (lds_void*)(buf + 1024 * (wave * kDmaPerWave + j0 + j)),
                                         16, 0, kNT);
      }
    }
  };
  auto prime = [&]() {
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    barrier_in_flight<kDmaPerWave>();
  };

  // ---- per-lane LDS addresses of the two read patterns
  const int sw_lj = swz(lj);
  const int li = lane & 15, g = lane >> 4;
  const int r1 = 4 * half + (li >> 2);                 // token of k elements 0..3 (+16 kk, +8)
  const int c0 = 2 * (g & 1) + ((li >> 1) & 1);        // chunk of dims 32 n + 16 (g&1) + 4 (li&3)
  const int sw_r1 = swz(r1);                           // rows r1 + 8, r1 + 16 share it

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

  auto step = [&](auto buf_id, int tix, int par) {
    constexpr int BI = decltype(buf_id)::value;
    if (BI == 1 && threadIdx.x == 0) restart_vote[par ^ 1] = 0;  // read by all before this tile
    const char* cur = BI == 0 ? tile0 : BI == 1 ? tile1 : tile2;
    issue(std::integral_constant<int, (BI + 2) % 3>{}, tix + 2);

    // Per-lane byte offsets into the tile, made opaque here so that the
    // compiler keeps six of them per tile instead of an address per read.
    // A operand of the scores: row lj, chunk c = 2 ks + half, stored at slot
    // 8 (c / 8) + ((c % 8) ^ f(lj)): offset so[ks % 4] + 128 (ks / 4).
    // B operand of P.V: rows r1 (+8) + 16 kk, chunk c = 4 n + c0, stored at
    // 8 (c / 8) + ((c % 8) ^ f(r1)): offset vo[n % 2] + 128 (n / 2) + ...
    uint32_t so[4], vo[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      so[j] = lj * (kDq * 2) + 16 * (((2 * j) | half) ^ sw_lj);
      asm volatile("" : "+v"(so[j]));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      vo[j] = r1 * (kDq * 2) + 16 * ((4 * j + c0) ^ sw_r1) + 8 * (li & 1);
      asm volatile("" : "+v"(vo[j]));
    }

    // S^T (32 tokens x 32 heads): lane holds head lj, tokens 8(v/4) + 4 half + v%4
    auto aread = [&](int ks) -> bf16x8_t {
      return *(const bf16x8_t*)(cur + so[ks & 3] + 128 * (ks >> 2));
    };
    f32x16_t s;
    {
      bf16x8_t ring[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) ring[j] = aread(j);
      asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                   : "=&v"(s) : "v"(ring[0]), "v"(qf[0]));
      ring[0] = aread(3);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 1; ks < kKSteps; ++ks) {
        asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+v"(s) : "v"(ring[ks % 3]), "v"(qf[ks]));
        if (ks + 3 < kKSteps) ring[ks % 3] = aread(ks + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the scores are read by ordinary code next: let the last MFMA retire
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
    }

    // online softmax for head lj (lanes lj and lj + 32 share the head)
    const uint32_t* rt = rows + tix * kTile + 4 * half;
    float mx = NEG_INF;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint4 e = *(const uint4*)(rt + 8 * q4);
      const uint32_t ev[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = 4 * q4 + u;
        s[v] = (ev[u] & kPad) ? NEG_INF : s[v] * a.scale_log2;
        mx = fmaxf(mx, s[v]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m_seen = fmaxf(m_seen, mx);
    // a head's first scores set its reference (its O is still zero); a later
    // score past the reference by more than kTau asks for a restart
    if (m_run != NEG_INF && mx > m_run + kTau) restart_vote[par] = 1;
    if (m_run == NEG_INF) m_run = mx;
    const float mu = m_run == NEG_INF ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = fast_exp2(s[v] - mu);
      psum += s[v];
    }
    l_run += psum;

    // O += P . V over two 16-token k-steps; V read transposed from the tile
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 pa;
      pa.x = pack_bf16x2(s[8 * kk + 0], s[8 * kk + 1]);
      pa.y = pack_bf16x2(s[8 * kk + 2], s[8 * kk + 3]);
      pa.z = pack_bf16x2(s[8 * kk + 4], s[8 * kk + 5]);
      pa.w = pack_bf16x2(s[8 * kk + 6], s[8 * kk + 7]);
      const bf16x8_t pab = __builtin_bit_cast(bf16x8_t, pa);
      auto vread = [&](int n) -> bf16x8_t {
        // dims 32 n + 16 (g&1) + 4 (li&3) .. + 3 of tokens r1 + 16 kk and r1 + 16 kk + 8
        const uint32_t off = vo[n & 1] + 128 * (n >> 1) + 16 * kk * (kDq * 2);
        const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(cur + off));
        const bf16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(cur + off + 8 * kDq * 2));
        return __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8_t vr[3];
#pragma unroll
      for (int n = 0; n < 3; ++n) vr[n] = vread(n);
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) {
        asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(acc[n]) : "v"(pab), "v"(vr[n % 3]));
        if (n + 3 < kNTiles) vr[n % 3] = vread(n + 3);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // tile tix + 1 complete in LDS for every wave (only tile tix + 2 may
    // still be in flight), tile tix free for reuse
    barrier_in_flight<kDmaPerWave>();
  };

  // the loop body has no branches around tiles: a tile past the split is
  // all padding (P = 0), and two tiles are always in flight
  if (n_groups > 0) {
    prime();
    for (int it = 0; it < n_groups; ++it) {
      const int par = it & 1;
      step(std::integral_constant<int, 0>{}, 3 * it, par);
      step(std::integral_constant<int, 1>{}, 3 * it + 1, par);
      step(std::integral_constant<int, 2>{}, 3 * it + 2, par);
      if (restart_vote[par]) {
        // some head's maximum jumped: redo the split with every head's
        // reference at the largest score it has seen (each restart raises a
        // reference by more than kTau, so restarts are few)
        barrier_in_flight<0>();  // every wave has read the vote
        if (threadIdx.x == 0) restart_vote[0] = restart_vote[1] = 0;
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);  // in-flight MFMAs retire first
        zero_acc();
        m_run = m_seen;
        l_run = 0.f;
        prime();
        it = -1;
      }
    }
    wait_vmcnt<0>();  // the two prefetches past the end land before the workgroup ends
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
  mla_split_kernel<SPARSE, PAGED, NW><<<grid, block, 0, s>>>(a);
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
  return mla_heads_per_workgroup(a.H) == 128 ? launch_nw<4>(a, s) : launch_nw<2>(a, s);
}

}  // namespace dattn
