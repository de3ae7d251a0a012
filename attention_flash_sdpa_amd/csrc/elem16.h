// 16-bit input elements of the matrix-core kernels: bf16 or fp16.  Both share
// every data movement (2-byte elements, the same LDS layouts and transposing
// reads); only the matrix op, the packing of probabilities and the row-sum dot
// product differ, and these overloads pick them by element type.
#pragma once
#include <hip/hip_runtime.h>

namespace sdpa {

template <typename E>
struct Vec16 {
  typedef E x2 __attribute__((ext_vector_type(2)));
  typedef E x4 __attribute__((ext_vector_type(4)));
  typedef E x8 __attribute__((ext_vector_type(8)));
};
typedef float f32x16_e __attribute__((ext_vector_type(16)));

// D[32x32] += A[32x16] . B[16x32] with fp32 accumulation.
__device__ __forceinline__ f32x16_e mfma32(Vec16<__bf16>::x8 a, Vec16<__bf16>::x8 b, f32x16_e c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_e mfma32(Vec16<_Float16>::x8 a, Vec16<_Float16>::x8 b, f32x16_e c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// acc + v[0] + v[1] in one dot-product instruction.
__device__ __forceinline__ float dot2_ones(Vec16<__bf16>::x2 v, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(v, (Vec16<__bf16>::x2){(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}
__device__ __forceinline__ float dot2_ones(Vec16<_Float16>::x2 v, float acc) {
  return __builtin_amdgcn_fdot2(v, (Vec16<_Float16>::x2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
}

}  // namespace sdpa
