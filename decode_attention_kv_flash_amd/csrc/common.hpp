// Device helpers shared by the dattn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 stored as raw 16-bit patterns; widening to fp32 is exact.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// fp32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32: round to
// nearest even, NaN preserved).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Pairs of bf16 halves from two dwords: (lo(a), lo(b)) and (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// DPP lane permutes inside a row of 16 lanes.
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {8, 16, 32, 64}); every lane of the
// group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  if constexpr (N >= 16) x += dpp_f32<0x140>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_f32<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// 16-byte load of data read once (K/V or latent rows): the nontemporal hint
// keeps the stream from displacing reused lines in the caches.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  typedef unsigned __attribute__((ext_vector_type(4))) u32x4;
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Order-preserving unsigned key of an fp32 score (-0.0 folded onto +0.0):
// a > b as floats exactly when key(a) > key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// LDS histogram add of bin d for the lanes with act set; a wave whose active
// lanes share one bin adds once (scores often crowd into one top byte).
__device__ __forceinline__ void hist_add(uint32_t* h, bool act, uint32_t d) {
  const uint64_t am = __ballot(act);
  if (am == 0) return;
  const int first = __ffsll((long long)am) - 1;
  const uint32_t d0 = __shfl(d, first);
  const uint64_t same = __ballot(act && d == d0);
  if (same == am) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&h[d0], (uint32_t)__popcll(am));
  } else if (act) {
    atomicAdd(&h[d], 1u);
  }
}

// exp2 of a value that may be -inf (gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs packed in 32 bits; the products
// of bf16 values are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// a.lo*b.lo + a.hi*b.hi with nothing to accumulate: the three-operand form
// with an inline zero (the compiler's choice, the accumulating two-operand
// form, would first move a zero into the destination).
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// ---- direct-to-LDS copies and the waits around them

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
// (The signal fences keep the compiler from moving memory accesses across it.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier that leaves the newest N tile copies of this wave in
// flight: wait until at most N vector-memory operations are outstanding and
// every LDS access of this wave is done, then s_barrier.  The signal fences
// keep the compiler from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void barrier_in_flight() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One wave-wide 16-byte-per-lane copy from global memory into LDS at
// lds_dst + 16 * lane (lds_dst uniform).  M0 carries the LDS address and is
// restored afterwards.
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds_dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"((uint64_t)(uintptr_t)src), "s"(lds_dst)
      : "memory");
}

}  // namespace dattn
