// Device helpers shared by the HIP kernels of libpkv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) short v4i16;

// Element type tags (match pkv_dtype).
enum Dt : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)x;
}

// Decode one element of storage type DT (given as raw bits) to float.
template <int DT>
__device__ __forceinline__ float elem_to_f32(uint32_t bits);
template <>
__device__ __forceinline__ float elem_to_f32<kF32>(uint32_t bits) { return __uint_as_float(bits); }
template <>
__device__ __forceinline__ float elem_to_f32<kF16>(uint32_t bits) { return f16_bits_to_f32(bits); }
template <>
__device__ __forceinline__ float elem_to_f32<kBF16>(uint32_t bits) { return bf16_bits_to_f32(bits); }
template <>
__device__ __forceinline__ float elem_to_f32<kFP8>(uint32_t bits) {
  // Hardware OCP E4M3 -> f32 conversion (exact: every E4M3 value is a float).
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)bits, false);
  return v[0];
}

// Round a float to bf16 bits, nearest-even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// OCP E4M3 encoding of a binary32, round-to-nearest-even, saturating finite
// overflow (and infinities) to +-448, NaN -> 0x7F; the sign of zero is kept.
// Written from the format: 4 exponent bits (bias 7), 3 mantissa bits,
// subnormals m/8 * 2^-6, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;           // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;   // |y| >= 448 (inf included)
  if (a < 0x3c800000u) {                       // |y| < 2^-6: multiples of 2^-9
    // |y| * 512 is exact; rint rounds half to even, which is an even code.
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)m;                 // m == 8 is the smallest normal, code 0x08
  }
  const uint32_t e = (a >> 23) - 120u;         // binary32 exponent - 127 + 7
  const uint32_t mant = a & 0x7fffffu;
  uint32_t code = (e << 3) | (mant >> 20);
  const uint32_t rest = mant & 0xfffffu;       // the 20 bits dropped
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) code += 1u;  // may carry into e
  return sign | code;                          // stays <= 0x7E because |y| < 448
}

// Wave-wide helpers (wave64).
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Compiler-only memory barrier: keeps the compiler from moving memory
// accesses across it.  A wave's LDS instructions execute in issue order, so
// within one wave this is all that lane-to-lane LDS exchange needs.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

}  // namespace pkv
