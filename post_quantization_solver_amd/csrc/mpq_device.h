// Device-side helpers shared by the MPQ kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

#define MPQ_WAVE 64

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// float -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f2bf_bits(float x) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)x);
}
// Two floats -> packed bfloat16 pair (x in the low half), round to nearest even.
__device__ __forceinline__ uint32_t f2bf_pack(float x, float y) {
  v2bf v = {(__bf16)x, (__bf16)y};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf_bits2f(uint32_t b) { return __uint_as_float(b << 16); }

// Split a float32 into three bfloat16 terms whose sum reproduces it to
// about 2^-24 relative (each term rounds the remainder of the previous).
__device__ __forceinline__ void split3_bf16(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = f2bf_bits(x);
  float r1 = x - bf_bits2f(h);
  m = f2bf_bits(r1);
  float r2 = r1 - bf_bits2f(m);
  l = f2bf_bits(r2);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xffffu) | (hi16 << 16); }

// A caller-supplied code used as a table index: codes outside [0, K) read
// entry 0 instead (the kernels that read such codes make their rows NaN, so
// nothing is decided from the stand-in).
__device__ __forceinline__ int safe_code(int c, int K) { return (unsigned)c < (unsigned)K ? c : 0; }

// This thread's wave within the workgroup, as a wave-uniform (scalar) value:
// the compiler then keeps the addresses derived from it in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Cross-lane helpers (full wave64).
__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ uint32_t shfl_i(uint32_t v, int src) { return (uint32_t)__shfl((int)v, src, 64); }
__device__ __forceinline__ double shfl_d(double v, int src) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = shfl_i((uint32_t)u, src), hi = shfl_i((uint32_t)(u >> 32), src);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// DPP lane patterns within a 16-lane row: quad_perm [1,0,3,2] (xor 1) and
// [2,3,0,1] (xor 2), row_half_mirror (lane i <-> 7 - i of each 8) and
// row_mirror (i <-> 15 - i).  In a reduction step whose lane quads (or halves)
// already hold one value each, the mirrors pair the same quads (halves) as
// xor 4 (xor 8), so a butterfly over them gives the xor butterfly's values.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int lo = dpp_i<CTRL>((int)(uint32_t)b);
  const int hi = dpp_i<CTRL>((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// MFMA wrappers.  16x16 output layout (all dtypes): lane l holds rows
// 4*(l/16) + v (v = 0..3) of column l % 16.
__device__ __forceinline__ v4f mfma_f32_16x16x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v4u a, v4u b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// The bf16 pairs (-1, 0) and (0, -1) as 32-bit words held in VGPRs.  They are
// moved in as literals: the compiler would otherwise encode (-1, 0) as the
// inline constant -1.0, which v_dot2c_f32_bf16 does not read as that pair.
struct DotMasks {
  uint32_t lo, hi;
};
__device__ __forceinline__ DotMasks dot_masks() {
  DotMasks d;
  asm volatile("v_mov_b32 %0, 0xbf80" : "=v"(d.lo));
  asm volatile("v_mov_b32 %0, 0xbf800000" : "=v"(d.hi));
  return d;
}
// x - (element 0 or 1 of the bf16 pair h), exact whenever the difference is a
// float32 (h rounded from x): one v_dot2_f32_bf16 with the pair (-1, 0) / (0, -1).
__device__ __forceinline__ float sub_bf16_lo(float x, uint32_t h, const DotMasks& dm) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, h), __builtin_bit_cast(v2bf, dm.lo), x, false);
}
__device__ __forceinline__ float sub_bf16_hi(float x, uint32_t h, const DotMasks& dm) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, h), __builtin_bit_cast(v2bf, dm.hi), x, false);
}
