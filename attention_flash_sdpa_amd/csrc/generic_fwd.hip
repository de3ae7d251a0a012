// Generic fused attention on the vector ALUs: any head_dim up to 128, fp32 or
// bf16 inputs, every bias kind.  It serves the fp32 path and shapes that the
// MFMA kernels do not cover.
//
// One wave per block, one query row per lane.  K/V tiles of 32 keys are staged
// through LDS as fp32; each lane keeps its query row and output accumulator in
// registers and runs the online softmax (running max m, running sum l; the
// accumulator is rescaled by exp(m_old - m_new) when the max grows), so no
// score row is ever stored.
//
// Definition followed ([Axon PR 650] "Axon.Layers.scaled_dot_product_attention/4",
// description; [mlx-examples issue 1451] "segment_anything: fuse attention with
// mx.fast.scaled_dot_product_attention", body):
//   z_ij = scale * q_i . k_j + bias_ij,  O_i = sum_j softmax_j(z_i.) v_j.
#include "common.h"

namespace sdpa {

// Mask families, one kernel instance each (small code per instance: with few
// waves per CU, instruction fetch dominates large kernels).
enum GenericFamily { GF_NONE = 0, GF_INDEX = 1, GF_TENSOR = 2, GF_RELPOS = 3 };

template <typename TIN, int DMAX, int GF>
__global__ __launch_bounds__(64) void generic_fwd_kernel(FwdParams p) {
  constexpr int BK = 32;
  __shared__ float ks[BK][DMAX];
  __shared__ float vs[BK][DMAX];
  __shared__ float zs[BK][64];        // this tile's scores, one column per lane
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.z, h = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t i = i0 + lane;
  const bool live = i < p.Tq;
  const int D = (int)p.D;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const TIN* qp = (const TIN*)p.q + b * p.q_sb + h * p.q_sh + (live ? i : 0) * p.q_st;
  const TIN* kp = (const TIN*)p.k + b * p.k_sb + hk * p.k_sh;
  const TIN* vp = (const TIN*)p.v + b * p.k_sb + hk * p.k_sh;

  float qr[DMAX], acc[DMAX];
#pragma unroll
  for (int c = 0; c < DMAX; ++c) {
    qr[c] = (c < D && live) ? to_f32(qp[c]) : 0.0f;
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  // Key range any row of this block can see.
  int64_t lo = 0, hi = p.Tkv;
  const int64_t ilast = (i0 + 63 < p.Tq - 1) ? i0 + 63 : p.Tq - 1;
  if (GF == GF_INDEX) {
    hi = ilast + p.offset + 1;
    if (hi > p.Tkv) hi = p.Tkv;
    if (p.bias == BIAS_SLIDING) {
      lo = i0 + p.offset - p.window + 1;
      if (lo < 0) lo = 0;
    }
  }
  const float* th = nullptr;
  const float* tw = nullptr;
  if (GF == GF_RELPOS) {
    th = p.term_h + ((b * p.Hq + h) * p.Tq + (live ? i : 0)) * p.grid_h;
    tw = p.term_w + ((b * p.Hq + h) * p.Tq + (live ? i : 0)) * p.grid_w;
  }

  for (int64_t j0 = lo; j0 < hi; j0 += BK) {
    __syncthreads();
    for (int e = lane; e < BK * DMAX; e += 64) {
      const int jj = e / DMAX, c = e % DMAX;
      const int64_t j = j0 + jj;
      const bool ok = j < hi && c < D;
      ks[jj][c] = ok ? to_f32(kp[j * p.k_st + c]) : 0.0f;
      vs[jj][c] = ok ? to_f32(vp[j * p.k_st + c]) : 0.0f;
    }
    __syncthreads();
    const int nk = (int)((hi - j0 < BK) ? hi - j0 : BK);
    float tmax = -INFINITY;
#pragma unroll 2
    for (int jj = 0; jj < nk; ++jj) {
      const int64_t j = j0 + jj;
      float d = 0.0f;
#pragma unroll
      for (int c = 0; c < DMAX; ++c) d = fmaf(qr[c], ks[jj][c], d);
      float z = d * p.scale;
      bool ok = live;
      if (GF == GF_INDEX) ok = ok && index_allowed(p.bias, i, j, p.offset, p.window);
      if (GF == GF_RELPOS && ok) z += th[j / p.grid_w] + tw[j % p.grid_w];
      if (GF == GF_TENSOR && ok) z += tensor_mask_bias(p, b, h, i, j);
      z = ok ? z : -INFINITY;
      zs[jj][lane] = z;
      tmax = fmaxf(tmax, z);
    }
    if (tmax > m) {             // the running max grows: rescale what has been summed
      const float corr = (m == -INFINITY) ? 0.0f : expf(m - tmax);
      l *= corr;
#pragma unroll
      for (int c = 0; c < DMAX; ++c) acc[c] *= corr;
      m = tmax;
    }
    if (m != -INFINITY) {
#pragma unroll 2
      for (int jj = 0; jj < nk; ++jj) {
        const float z = zs[jj][lane];
        const float pj = (z == -INFINITY) ? 0.0f : expf(z - m);
        l += pj;
#pragma unroll
        for (int c = 0; c < DMAX; ++c) acc[c] = fmaf(pj, vs[jj][c], acc[c]);
      }
    }
  }
  if (!live) return;
  const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
  const int64_t ob = b * p.q_sb + h * p.q_sh + i * p.q_st;
  if (p.out_dtype == 0) {
    float* op = (float*)p.o + ob;
#pragma unroll
    for (int c = 0; c < DMAX; ++c) if (c < D) op[c] = acc[c] * inv;
  } else {
    __bf16* op = (__bf16*)p.o + ob;
#pragma unroll
    for (int c = 0; c < DMAX; ++c) if (c < D) op[c] = (__bf16)(acc[c] * inv);
  }
  if (p.lse) p.lse[(b * p.Hq + h) * p.Tq + i] = (l > 0.0f) ? m + logf(l) : -INFINITY;
}

template <typename TIN, int DMAX>
static void launch_dim(const FwdParams& p, dim3 grid, hipStream_t s) {
  switch (p.bias) {
    case BIAS_NONE: hipLaunchKernelGGL((generic_fwd_kernel<TIN, DMAX, GF_NONE>), grid, dim3(64), 0, s, p); break;
    case BIAS_CAUSAL:
    case BIAS_SLIDING: hipLaunchKernelGGL((generic_fwd_kernel<TIN, DMAX, GF_INDEX>), grid, dim3(64), 0, s, p); break;
    case BIAS_RELPOS: hipLaunchKernelGGL((generic_fwd_kernel<TIN, DMAX, GF_RELPOS>), grid, dim3(64), 0, s, p); break;
    default: hipLaunchKernelGGL((generic_fwd_kernel<TIN, DMAX, GF_TENSOR>), grid, dim3(64), 0, s, p); break;
  }
}

template <typename TIN>
static hipError_t launch_typed(const FwdParams& p, hipStream_t s) {
  dim3 grid((unsigned)((p.Tq + 63) / 64), (unsigned)p.Hq, (unsigned)p.B);
  if (p.D <= 16) launch_dim<TIN, 16>(p, grid, s);
  else if (p.D <= 32) launch_dim<TIN, 32>(p, grid, s);
  else if (p.D <= 64) launch_dim<TIN, 64>(p, grid, s);
  else launch_dim<TIN, 128>(p, grid, s);
  return hipGetLastError();
}

hipError_t launch_generic_fwd(const FwdParams& p, hipStream_t s) {
  return p.dtype == 0 ? launch_typed<float>(p, s) : launch_typed<__bf16>(p, s);
}

}  // namespace sdpa
