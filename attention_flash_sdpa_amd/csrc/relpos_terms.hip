// Decomposed rel-pos terms of SAM's attention ([mlx-examples issue 1451]
// "segment_anything: fuse attention with mx.fast.scaled_dot_product_attention",
// body: add_decomposed_rel_pos; [Candle PR 3280] "feat(metal): SDPA with
// Relative Positional Embeddings & LayerNorm Stability", Key Changes: term_h
// and term_w):
//   term_h[b,h,i,y] = sum_c q[b,h,i,c] * rel_pos_h[row(i) - y + grid_h - 1, c]
//   term_w[b,h,i,x] = sum_c q[b,h,i,c] * rel_pos_w[col(i) - x + grid_w - 1, c]
//
// One workgroup per (b, h, grid row).  The grid_w queries of one grid row share
// a single gathered rel_pos_h block, so term_h for the row is the small product
// Q_row [grid_w x D] . Rh_rows^T [D x grid_h]; term_w for query (row, col) uses
// the rel_pos_w rows col - x + grid_w - 1.  The query rows and both gathered
// table blocks are staged in LDS as fp32 and every output is one fp32 dot
// product of length D.  Query rows are staged in LDS as fp32; the (small)
// tables are read through the cache.
#include "common.h"

namespace sdpa {

template <typename TIN>
__global__ __launch_bounds__(256) void relpos_terms_kernel(TermsParams p) {
  extern __shared__ float smem[];
  const int gh = p.grid_h, gw = p.grid_w;
  const int D = (int)p.D;
  const int DP = D + 1;                        // padded row pitch against bank conflicts
  float* qs = smem;                            // [gw][DP]
  const int64_t row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const TIN* q = (const TIN*)p.q + b * p.q_sb + h * p.q_sh;
  const TIN* rh = (const TIN*)p.rel_h;
  const TIN* rw = (const TIN*)p.rel_w;
  for (int e = threadIdx.x; e < gw * D; e += blockDim.x) {
    const int t = e / D, c = e % D;
    qs[t * DP + c] = to_f32(q[(row * gw + t) * p.q_st + c]);
  }
  __syncthreads();
  const int64_t base = (b * p.H + h) * p.T + row * gw;   // first query of this grid row
  // term_h: [gw queries][gh]
  for (int e = threadIdx.x; e < gw * gh; e += blockDim.x) {
    const int t = e / gh, y = e % gh;
    const float* a = qs + t * DP;
    const TIN* r = rh + (row - y + gh - 1) * D;
    float acc = 0.0f;
    for (int c = 0; c < D; ++c) acc = fmaf(a[c], to_f32(r[c]), acc);
    p.term_h[(base + t) * gh + y] = acc;
  }
  // term_w: [gw queries][gw]
  for (int e = threadIdx.x; e < gw * gw; e += blockDim.x) {
    const int t = e / gw, x = e % gw;
    const float* a = qs + t * DP;
    const TIN* r = rw + (int64_t)(t - x + gw - 1) * D;
    float acc = 0.0f;
    for (int c = 0; c < D; ++c) acc = fmaf(a[c], to_f32(r[c]), acc);
    p.term_w[(base + t) * gw + x] = acc;
  }
}

hipError_t launch_relpos_terms(const TermsParams& p, hipStream_t s) {
  const size_t lds = sizeof(float) * (size_t)(p.D + 1) * (size_t)p.grid_w;
  dim3 grid((unsigned)p.grid_h, (unsigned)p.H, (unsigned)p.B);
  if (p.dtype == 0) hipLaunchKernelGGL(relpos_terms_kernel<float>, grid, dim3(256), lds, s, p);
  else if (p.dtype == 2) hipLaunchKernelGGL(relpos_terms_kernel<_Float16>, grid, dim3(256), lds, s, p);
  else hipLaunchKernelGGL(relpos_terms_kernel<__bf16>, grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace sdpa
