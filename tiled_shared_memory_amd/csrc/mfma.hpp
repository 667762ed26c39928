// gfx950 matrix-core helpers: vector types, MFMA wrappers and operand layouts.
//
// The blocked product is a dense contraction, so its inner step runs on the
// CDNA4 matrix cores (MFMA).  Operand and accumulator lane layouts used by the
// kernels, for a 64-lane wavefront (lane l):
//
//   v_mfma_f32_32x32x16_{f16,bf16}:  D(32x32) += A(32x16) * B(16x32)
//     A operand: 8 x 16-bit per lane = A[m = l%32][k = 8*(l/32) + 0..7]
//     B operand: 8 x 16-bit per lane = B[k = 8*(l/32) + 0..7][n = l%32]
//     D: 16 floats per lane, register r holds D[m][n] with
//        n = l%32,  m = 8*(r/4) + 4*(l/32) + r%4
//
//   v_mfma_f32_16x16x32_{f16,bf16}:  D(16x16) += A(16x32) * B(32x16)
//     A operand: A[m = l%16][k = 8*(l/16) + 0..7]
//     B operand: B[k = 8*(l/16) + 0..7][n = l%16]
//     D: 4 floats per lane, register r holds D[m = 4*(l/16) + r][n = l%16]
//
// Only the pairing of k between the A and B operands matters for the sum, so
// any k order inside a 16- or 32-deep step is valid as long as both operands
// use the same one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

template <bool BF16>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
}

// float32 -> f16, round to nearest even (the hardware default rounding mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// Store one accumulator value into row-major C if it lies inside M x N.
template <bool OUT_F16>
__device__ __forceinline__ void store_masked(void *C, int64_t ldc, int64_t M, int64_t N, int64_t row, int64_t col,
                                             float v) {
  if (row < M && col < N) {
    if constexpr (OUT_F16)
      reinterpret_cast<uint16_t *>(C)[row * ldc + col] = f32_to_f16_bits(v);
    else
      reinterpret_cast<float *>(C)[row * ldc + col] = v;
  }
}

}  // namespace tsm
