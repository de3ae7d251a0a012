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

// Orders this wave's LDS accesses before and after it: a wave's LDS
// operations execute in issue order, and the fences keep the compiler from
// moving them across.  Enough where only the wave's own lanes share the words.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait states after matrix ops whose results the vector ALU reads next.  A
// vector read of a matrix op's result needs wait states (the 8-pass 32x32x16
// op: at least 11) that the hardware does not enforce; the compiler inserts
// them, but counts them along the first control-flow path it finds back to
// the op.  Where an exec-mask branch around lane-divergent code sits between
// the op and the read, the branch-taken path can then reach the read a few
// instructions after the op, and the read sees registers the op has not yet
// written.  This fence takes the results as operands where they are (the
// accumulation registers, so it needs no copy), so the ops that produce them
// come before it and every read of them after it, with 14 wait states in
// between on every path.  For kernels whose matrix ops accumulate in AGPRs.
typedef float f32x16_fence __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void mfma_drain(f32x16_fence& a) { asm volatile("s_nop 7\n\ts_nop 5" : "+a"(a)); }
__device__ __forceinline__ void mfma_drain(f32x16_fence& a, f32x16_fence& b) {
  asm volatile("s_nop 7\n\ts_nop 5" : "+a"(a), "+a"(b));
}

}  // namespace sdpa
