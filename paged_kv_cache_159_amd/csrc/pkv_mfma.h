// MFMA (matrix core) wrappers for gfx950 used by the grouped decode and the
// prefill kernels, on 16-bit operands held as raw bits.
//
// Operand layouts (64 lanes, lane l, row/column index l % 16, lane group
// g = l / 16), measured on the device:
//   16x16x32 (K = 32): A lane l holds A[l%16][8g + e], B holds B[8g + e][l%16],
//                      e = 0..7 (16 bytes per lane);
//   16x16x16 (K = 16): the same with 4g + e, e = 0..3 (8 bytes per lane);
//   accumulator (both): lane l holds C[4g + v][l%16], v = 0..3.
#pragma once

#include "pkv_device.h"

namespace pkv {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;

template <> struct Mfma<F16> {
  // C += A B with A 16x32, B 32x16 (8 elements per lane each).
  static __device__ __forceinline__ f4_t k32(uint4 a, uint4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
  }
  // C += A B with A 16x16, B 16x16 (4 elements per lane each).
  static __device__ __forceinline__ f4_t k16(uint2 a, uint2 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a),
                                                 __builtin_bit_cast(h4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)x);
  }
};

template <> struct Mfma<BF16> {
  static __device__ __forceinline__ f4_t k32(uint4 a, uint4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                   __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4_t k16(uint2 a, uint2 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a),
                                                     __builtin_bit_cast(s4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint32_t x) { return __uint_as_float(x << 16); }
};

// Max / sum over the 4 lane groups of an MFMA tile (lanes l, l^16, l^32,
// l^48: one column of the accumulator) with gfx950's row-swap instructions
// instead of LDS permutes. With both operands equal to x, v_permlane16_swap
// returns x's even 16-lane rows in both rows of each pair in one result and
// its odd rows in the other (measured on the device), so combining the two
// gives op(x[l], x[l^16]) in every lane; v_permlane32_swap does the same
// across the two 32-lane halves. The two inputs of each combine are taken in
// the same order in every lane, so all lanes get bit-identical results.
__device__ __forceinline__ float lane_group4_max(float v) {
  const unsigned x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned y = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float lane_group4_sum(float v) {
  const unsigned x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned y = __float_as_uint(s);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace pkv
