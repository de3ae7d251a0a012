// Device helpers shared by the HIP kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "internal.h"

namespace sdpa {

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }

// Load one element of an additive (F32/BF16) or boolean (uint8) mask and turn it
// into an additive bias: ADDITIVE adds the value, BOOL adds 0 (attend) or -inf.
__device__ __forceinline__ float tensor_mask_bias(const FwdParams& p, int64_t b, int64_t h, int64_t i, int64_t j) {
  const int64_t off = b * p.ms[0] + h * p.ms[1] + i * p.ms[2] + j * p.ms[3];
  if (p.bias == BIAS_BOOL) return ((const uint8_t*)p.mdata)[off] ? 0.0f : -INFINITY;
  if (p.mdtype == 0) return ((const float*)p.mdata)[off];
  return (float)((const __bf16*)p.mdata)[off];
}

// Index-mask test: causal (j <= i + offset) and sliding (i + offset - window < j <= i + offset).
__device__ __forceinline__ bool index_allowed(int bias, int64_t i, int64_t j, int64_t offset, int64_t window) {
  if (bias == BIAS_CAUSAL) return j <= i + offset;
  if (bias == BIAS_SLIDING) return j <= i + offset && j > i + offset - window;
  return true;
}

}  // namespace sdpa
