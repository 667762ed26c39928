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

// float32 -> bf16, round to nearest even (converted in hardware on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

// The epilogue every kernel applies to a float32 accumulator value before it
// is stored: an optional activation (the ACTIVATION meta-parameter of the Intel
// XPU Triton README's matmul signature, "Use Proper Type Annotations"), then
// the conversion to the output format.  Uniform across a launch.
struct Epilogue {
  int act;      // 0 none, 1 ReLU, 2 leaky ReLU
  float slope;  // leaky ReLU: the factor applied to negative values
  bool bf16;    // a 16-bit output is bf16 (else f16)

  __device__ __forceinline__ float apply(float v) const {
    if (act == 0) return v;
    return v > 0.f ? v : (act == 1 ? 0.f : v * slope);
  }
  __device__ __forceinline__ uint16_t to16(float v) const { return bf16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v); }
};

__device__ __forceinline__ Epilogue epilogue_of(const KernelArgs &p) { return Epilogue{p.act, p.slope, p.out_bf16 != 0}; }

// The same, copied into vector registers at once: for kernels whose scalar
// registers are the scarce ones (the values are uniform either way).
__device__ __forceinline__ Epilogue epilogue_in_vgprs(const KernelArgs &p) {
  int act, bf16;
  float slope;
  asm("v_mov_b32 %0, %1" : "=v"(act) : "s"(p.act));
  asm("v_mov_b32 %0, %1" : "=v"(slope) : "s"(p.slope));
  asm("v_mov_b32 %0, %1" : "=v"(bf16) : "s"(p.out_bf16));
  return Epilogue{act, slope, bf16 != 0};
}

// Four consecutive values of one row of C, at C (16 bytes of float32 or
// 8 bytes of 16-bit values; the callers keep the address aligned).
template <bool OUT16>
__device__ __forceinline__ void store4(void *C, const Epilogue &e, float v0, float v1, float v2, float v3) {
  v0 = e.apply(v0);
  v1 = e.apply(v1);
  v2 = e.apply(v2);
  v3 = e.apply(v3);
  if constexpr (OUT16) {
    u32x2 v;
    v[0] = (uint32_t)e.to16(v0) | ((uint32_t)e.to16(v1) << 16);
    v[1] = (uint32_t)e.to16(v2) | ((uint32_t)e.to16(v3) << 16);
    *reinterpret_cast<u32x2 *>(C) = v;
  } else {
    *reinterpret_cast<f32x4 *>(C) = f32x4{v0, v1, v2, v3};
  }
}

// Store one accumulator value into row-major C if it lies inside M x N.
template <bool OUT16>
__device__ __forceinline__ void store_masked(void *C, int64_t ldc, int64_t M, int64_t N, int64_t row, int64_t col,
                                             float v, const Epilogue &e) {
  if (row < M && col < N) {
    v = e.apply(v);
    if constexpr (OUT16)
      reinterpret_cast<uint16_t *>(C)[row * ldc + col] = e.to16(v);
    else
      reinterpret_cast<float *>(C)[row * ldc + col] = v;
  }
}

}  // namespace tsm
