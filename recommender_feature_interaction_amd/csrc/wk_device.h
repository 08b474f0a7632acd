// Device helpers shared by the Wukong HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even (NaN stays NaN): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8(l/16)..+7] and
// B[8(l/16)..+7][l%16]; it receives D[4(l/16)+t][l%16], t = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D(32x32) += A(32x16) * B(16x32).  Lane l supplies A[l%32][8(l/32)..+7] and
// B[8(l/32)..+7][l%32]; it receives D[8(r/4) + 4(l/32) + r%4][l%32], r = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Sum over the lanes l ^ mask for mask in [from, 32] (powers of two).
template <int FROM>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int m = FROM; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
// Sum over groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64):
// within a 16-lane row on the VALU with DPP (quad_perm for lanes l ^ 1 and
// l ^ 2, row_half_mirror and row_mirror to join the quads and then the two
// halves of the row), across rows with shuffles.  Every lane of a group ends
// with the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
template <int G>
__device__ __forceinline__ float group_sum_v(float v) {
  if constexpr (G >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  if constexpr (G >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  if constexpr (G >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (G >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (G >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Select 16-bit halves of two dwords (v_perm_b32): lo16(a) | lo16(b) << 16 ...
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// The shared-gate SwiGLU activation silu(v) * v = v^2 * logistic(v) with the
// hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each, no
// denormal range handling; the callers round the result to bf16).  For
// v < -88, exp(-v) overflows to +inf and the reciprocal gives 0, the value to
// bf16 precision.
__device__ __forceinline__ float silu_gate(float v) {
  return v * v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(v * -1.44269504088896341f));
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() is a
// workgroup release/acquire fence plus s_barrier, and on gfx9 the release
// half waits for every outstanding vector memory operation (global loads and
// stores included); this one waits for LDS traffic (lgkmcnt) only, so global
// prefetches and stores stay in flight across it.  Use it where waves share
// nothing but LDS.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier of an LDS ring filled by LDS DMA (buffer_load ... lds).
// The DMA writes count as outstanding LDS writes, so a release fence on LDS
// (lds_barrier) makes the compiler wait for every DMA in flight (vmcnt(0)),
// prefetches of later slots included, and the ring drains at every step.  The
// callers wait for their own DMAs of the slot about to be read with an explicit
// vmcnt count first; this barrier waits only for the wave's LDS operations
// (lgkmcnt(0)).  The asm's memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace wk
