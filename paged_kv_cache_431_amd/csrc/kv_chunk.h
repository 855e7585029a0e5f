// Eight consecutive elements of one cached row, moved with 16-byte (8-byte
// for FP8) accesses, and their conversion into an FP8 pool.  Shared by the
// scatter kernel and the decode step that appends the new token itself, so
// that both write the same bits.
#pragma once

#include "device_common.h"

namespace pkv {

typedef uint32_t c8_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t c8_u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Chunk8;  // 8 elements of storage type DT
template <>
struct Chunk8<kF32> {
  c8_u32x4 w[2];
};
template <>
struct Chunk8<kF16> {
  c8_u32x4 w;
};
template <>
struct Chunk8<kBF16> {
  c8_u32x4 w;
};
template <>
struct Chunk8<kFP8> {
  c8_u32x2 w;
};

template <int DT>
__device__ __forceinline__ Chunk8<DT> load8(const uint8_t* p) {
  Chunk8<DT> c;
  if constexpr (DT == kF32) {
    c.w[0] = reinterpret_cast<const c8_u32x4*>(p)[0];
    c.w[1] = reinterpret_cast<const c8_u32x4*>(p)[1];
  } else if constexpr (DT == kFP8) {
    c.w = *reinterpret_cast<const c8_u32x2*>(p);
  } else {
    c.w = *reinterpret_cast<const c8_u32x4*>(p);
  }
  return c;
}

template <int DT>
__device__ __forceinline__ void store8(uint8_t* p, const Chunk8<DT>& c) {
  if constexpr (DT == kF32) {
    reinterpret_cast<c8_u32x4*>(p)[0] = c.w[0];
    reinterpret_cast<c8_u32x4*>(p)[1] = c.w[1];
  } else if constexpr (DT == kFP8) {
    *reinterpret_cast<c8_u32x2*>(p) = c.w;
  } else {
    *reinterpret_cast<c8_u32x4*>(p) = c.w;
  }
}

template <int DT>
__device__ __forceinline__ float chunk_elem(const Chunk8<DT>& c, int e) {
  if constexpr (DT == kF32) {
    return __uint_as_float(c.w[e >> 2][e & 3]);
  } else {
    const uint32_t word = c.w[e >> 1];
    return elem_to_f32<DT>((e & 1) ? (word >> 16) : (word & 0xffffu));
  }
}

template <int IN>
__device__ __forceinline__ Chunk8<kFP8> quantize8(const Chunk8<IN>& c, float scale) {
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = f32_to_e4m3_sat(__fdiv_rn(chunk_elem<IN>(c, e), scale));
  Chunk8<kFP8> o;
  o.w = c8_u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
  return o;
}

}  // namespace pkv
