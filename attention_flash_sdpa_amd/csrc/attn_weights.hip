// Attention weights for `:return_attention_weights` ([Axon PR 650]
// "Axon.Layers.scaled_dot_product_attention/4", description): the weights
// that multiply V,
//   W~[b, h, i, j] = exp(scale * q_i . k_j + bias_ij - lse_i) * Z_ij
// rebuilt from the forward pass's row log-sum-exp (so the row normalisation
// is the forward pass's own), with Z the dropout factor when keep bits are
// given and 1 otherwise.  Written as fp32 [B, Hq, Tq, Tkv].  This is a debug
// output: the T_q x T_kv write bounds it, and it runs on the vector ALUs.
//
// One workgroup per 64 x 64 block of one (batch, head); the Q and K blocks
// are staged through LDS as fp32 and each thread forms a 4 x 4 patch, stored
// as 16-byte rows (a wavefront covers four full 256-byte output rows).
#include "common.h"

namespace sdpa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename TIN, int DMAX>
__global__ __launch_bounds__(256) void attn_weights_kernel(FwdParams p, float* out) {
  constexpr int P = DMAX + 1;              // odd pitch: conflict-free column reads
  __shared__ float qs[64 * P];
  __shared__ float ks[64 * P];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.z, b = bh / p.Hq, h = bh % p.Hq;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int D = (int)p.D;
  const TIN* qp = (const TIN*)p.q + b * p.q_sb + h * p.q_sh;
  const TIN* kp = (const TIN*)p.k + b * p.k_sb + hk * p.k_sh;
  for (int e = tid; e < 64 * DMAX; e += 256) {
    const int r = e / DMAX, c = e % DMAX;
    qs[r * P + c] = (i0 + r < p.Tq && c < D) ? to_f32(qp[(i0 + r) * p.q_st + c]) : 0.0f;
    ks[r * P + c] = (j0 + r < p.Tkv && c < D) ? to_f32(kp[(j0 + r) * p.k_st + c]) : 0.0f;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;  // rows 4 ty .. +3, keys 4 tx .. +3
  float acc[4][4] = {};
  for (int c = 0; c < DMAX; ++c) {
    float a[4], k4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = qs[(4 * ty + u) * P + c];
      k4[u] = ks[(4 * tx + u) * P + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], k4[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + 4 * ty + u;
    if (i >= p.Tq) continue;
    const float lse = p.lse[bh * p.Tq + i];
    const uint32_t* kr = p.keep ? p.keep + (bh * p.Tq + i) * p.keep_words : nullptr;
    float w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t j = j0 + 4 * tx + v;
      float z = acc[u][v] * p.scale;
      // conditions combined without short-circuit and applied before the exponential
      // (exp(-inf) = 0), so no score takes a branch of its own
      bool ok = (j < p.Tkv) & (lse != -INFINITY);
      if (p.bias == BIAS_CAUSAL) ok = ok & (j <= i + p.offset);
      if (p.bias == BIAS_SLIDING) ok = ok & (j <= i + p.offset) & (j > i + p.offset - p.window);
      if (p.bias == BIAS_ADDITIVE || p.bias == BIAS_BOOL) {
        if (ok) z += tensor_mask_bias(p, b, h, i, j);
      }
      float wv = __expf(ok ? z - lse : -INFINITY);
      if (kr) {      // the word index is clamped to the row, so the load needs no guard
        const uint32_t word = kr[min(j, p.Tkv - 1) >> 5];
        wv = (ok & (((word >> (j & 31)) & 1u) != 0u)) ? wv * p.keep_scale : 0.0f;
      }
      w[v] = wv;
    }
    float* orow = out + (bh * p.Tq + i) * p.Tkv + j0 + 4 * tx;
    if (j0 + 4 * tx + 3 < p.Tkv && (p.Tkv & 3) == 0) {
      *(f32x4*)orow = (f32x4){w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (j0 + 4 * tx + v < p.Tkv) orow[v] = w[v];
    }
  }
}

template <typename TIN>
hipError_t launch_t(const FwdParams& p, float* w, hipStream_t s) {
  dim3 grid((unsigned)((p.Tkv + 63) / 64), (unsigned)((p.Tq + 63) / 64), (unsigned)(p.B * p.Hq));
  if (p.D <= 32) hipLaunchKernelGGL((attn_weights_kernel<TIN, 32>), grid, dim3(256), 0, s, p, w);
  else if (p.D <= 64) hipLaunchKernelGGL((attn_weights_kernel<TIN, 64>), grid, dim3(256), 0, s, p, w);
  else hipLaunchKernelGGL((attn_weights_kernel<TIN, 128>), grid, dim3(256), 0, s, p, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_weights(const FwdParams& p, float* weights, hipStream_t s) {
  if (p.dtype == 0) return launch_t<float>(p, weights, s);
  return p.dtype == 2 ? launch_t<_Float16>(p, weights, s) : launch_t<__bf16>(p, weights, s);
}

}  // namespace sdpa
