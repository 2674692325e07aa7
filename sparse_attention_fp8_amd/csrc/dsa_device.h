// Device-side helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---------------------------------------------------------------- MFMA wrappers
// 16x16x128 fp8 (OCP e4m3) x fp8 -> fp32.  Operand layout: lane l holds row
// (l & 15) of its 16-row operand and a 32-byte run of the 128-long contraction
// selected by l >> 4; A and B use the same run selection, so the product covers
// the whole contraction.  Result: lane l holds D[4*(l>>4) + v][l & 15], v = 0..3.
// The block scales are neutral (E8M0 127 = 1.0).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x32 bf16 -> fp32.  Lane l holds 8 bf16 of row (l & 15) for the
// contraction slots 8*(l>>4) .. 8*(l>>4)+7; result layout as above.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- conversions
// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even; on
// gfx950 this is the single v_cvt_pk_bf16_f32 instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// max(x, 0) for an IEEE float as one integer max on its bits: non-negative floats
// order like their bit patterns and every negative float has a negative pattern.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0.0 maps like +0.0; NaN is not expected (callers canonicalise it first).
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;  // -0.0 -> +0.0
  uint32_t mask = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
  return u ^ mask;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (lane_id() == 0) ? 0ull : (~0ull >> (64 - lane_id()));
}

}  // namespace dsa
