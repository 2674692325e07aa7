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
// No block scales: with zero scale operands the compiler emits the unscaled
// v_mfma_f32_16x16x128_f8f6f4, which gives the same bits as neutral E8M0 scales
// (127 = 1.0) in one instruction word less (measured: identical prefill scores,
// ~3 % faster).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
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
// Cross-lane moves without LDS: DPP (row = 16 lanes) and the gfx950 permlane swaps.
// dpp<CTRL, ROWS>(x): lane i receives x from the lane CTRL names; lanes whose
// source lies outside the row, or whose row is not in ROWS, receive 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, true);
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;       // lane i <- 15 - i within each row
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142;      // row r <- lane 15 of row r - 1
constexpr int kDppBcast31 = 0x143;      // rows 2, 3 <- lane 31

// the two halves of {x[l & ~16], x[l | 16]} and {x[l & ~32], x[l | 32]}
__device__ __forceinline__ uint2 swap16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ uint2 swap32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return make_uint2(r[0], r[1]);
}

// x of lane l ^ 16 and of lane l ^ 32, through the permlane swaps
__device__ __forceinline__ float xor16(float x) {
  const uint2 r = swap16(__float_as_uint(x));
  return __uint_as_float((threadIdx.x & 16) ? r.x : r.y);
}
__device__ __forceinline__ float xor32(float x) {
  const uint2 r = swap32(__float_as_uint(x));
  return __uint_as_float((threadIdx.x & 32) ? r.x : r.y);
}

// Reduction over the whole wave with a commutative, associative op: every lane
// gets the result.  Each step pairs lanes that already hold equal partials, so a
// mirror permutation serves as well as an xor one.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_bits(uint32_t v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppMirror>(v));
  uint2 s = swap16(v);
  v = op(s.x, s.y);
  s = swap32(v);
  return op(s.x, s.y);
}
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_min(float v) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce_bits(v, [](uint32_t a, uint32_t b) { return a + b; });
}
// OR over each aligned group of 8 lanes (every lane of the group gets it)
__device__ __forceinline__ uint32_t or8(uint32_t v) {
  v |= dpp<kDppXor1>(v);
  v |= dpp<kDppXor2>(v);
  return v | dpp<kDppHalfMirror>(v);
}
// Inclusive prefix sum over the wave (lane l gets v[0] + ... + v[l]).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<kDppShr1>(v);
  v += dpp<kDppShr2>(v);
  v += dpp<kDppShr4>(v);
  v += dpp<kDppShr8>(v);
  v += dpp<kDppBcast15, 0xa>(v);
  v += dpp<kDppBcast31, 0xc>(v);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (lane_id() == 0) ? 0ull : (~0ull >> (64 - lane_id()));
}

}  // namespace dsa
