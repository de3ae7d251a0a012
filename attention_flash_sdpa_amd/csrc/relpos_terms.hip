// Decomposed rel-pos terms of SAM's attention ([mlx-examples issue 1451]
// "segment_anything: fuse attention with mx.fast.scaled_dot_product_attention",
// body: add_decomposed_rel_pos; [Candle PR 3280] "feat(metal): SDPA with
// Relative Positional Embeddings & LayerNorm Stability", Key Changes: term_h
// and term_w):
//   term_h[b,h,i,y] = sum_c q[b,h,i,c] * rel_pos_h[row(i) - y + grid_h - 1, c]
//   term_w[b,h,i,x] = sum_c q[b,h,i,c] * rel_pos_w[col(i) - x + grid_w - 1, c]
//
// The grid_w queries of one grid row share a single gathered rel_pos_h block,
// so term_h for the row is the small product Q_row [grid_w x D] . Rh_rows^T
// [D x grid_h]; term_w for query (row, col) uses the rel_pos_w rows
// col - x + grid_w - 1.  Every output is one fp32 dot product of length D.
#include "common.h"

namespace sdpa {

// One workgroup per (b, h, grid row): its grid_w queries, each handled by
// 256 / grid_w threads (or one thread per query and a loop when grid_w > 256).
// A thread keeps its query row in registers (fp32) and forms its share of that
// query's grid_h + grid_w dot products, reading each table row with 16-byte
// loads (the tables are small and stay in cache) where the rows allow it.
// LDS_TAB: the grid row's gh rows of rel_pos_h and all 2 gw - 1 rows of
// rel_pos_w are first staged in LDS in the input type, rows padded by 16
// bytes (consecutive rows start 16 bytes of banks apart), and read from there.
template <typename TIN, int DMAX, bool VEC, bool LDS_TAB>
__global__ __launch_bounds__(256) void relpos_terms_kernel(TermsParams p) {
  extern __shared__ __attribute__((aligned(16))) char tab_lds[];
  const int gh = p.grid_h, gw = p.grid_w;
  const int D = (int)p.D;
  const int64_t row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const TIN* qb = (const TIN*)p.q + b * p.q_sb + h * p.q_sh;
  const TIN* rh = (const TIN*)p.rel_h;
  const TIN* rw = (const TIN*)p.rel_w;
  int pitch = D;                       // elements between table rows
  if (LDS_TAB) {
    constexpr int EPP = 16 / sizeof(TIN);
    pitch = D + EPP;
    TIN* th_s = (TIN*)tab_lds;                        // rows row .. row + gh - 1 of rel_pos_h
    TIN* tw_s = th_s + gh * pitch;                    // rows 0 .. 2 gw - 2 of rel_pos_w
    const int cpr = D / EPP;                          // 16-byte chunks per row
    typedef TIN tin16 __attribute__((ext_vector_type(EPP)));
    for (int e = threadIdx.x; e < (gh + 2 * gw - 1) * cpr; e += 256) {
      const int r = e / cpr, c = (e % cpr) * EPP;
      const tin16 v = r < gh ? *(const tin16*)(rh + (row + r) * D + c) : *(const tin16*)(rw + (int64_t)(r - gh) * D + c);
      *(tin16*)(th_s + r * pitch + c) = v;
    }
    __syncthreads();
    rh = th_s - row * pitch;                          // so that row index t addresses rh + t * pitch
    rw = tw_s;
  }
  const int64_t base = (b * p.H + h) * p.T + row * gw;   // first query of this grid row
  const int tpq = gw >= 256 ? 1 : 256 / gw;              // threads per query
  const int part = threadIdx.x % tpq;
  for (int t = threadIdx.x / tpq; t < gw; t += 256 / tpq) {
    float qr[DMAX];
    const TIN* qrow = qb + (row * gw + t) * p.q_st;
    if (VEC && (p.q_st * sizeof(TIN)) % 16 == 0 && ((uintptr_t)qb & 15) == 0) {
      constexpr int EPP = 16 / sizeof(TIN);
      typedef TIN tin16 __attribute__((ext_vector_type(EPP)));
#pragma unroll
      for (int c = 0; c < DMAX; c += EPP) {
        const tin16 v = (c < D) ? *(const tin16*)(qrow + c) : (tin16){};
#pragma unroll
        for (int e = 0; e < EPP; ++e) qr[c + e] = to_f32(v[e]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < DMAX; ++c) qr[c] = (c < D) ? to_f32(qrow[c]) : 0.0f;
    }
    auto dot = [&](const TIN* r) -> float {
      float acc = 0.0f;
      if (VEC) {
        constexpr int EPP = 16 / sizeof(TIN);
        typedef TIN tin16 __attribute__((ext_vector_type(EPP)));
#pragma unroll
        for (int c = 0; c < DMAX; c += EPP) {
          if (c < D) {
            const tin16 v = *(const tin16*)(r + c);
#pragma unroll
            for (int e = 0; e < EPP; ++e) acc = fmaf(qr[c + e], to_f32(v[e]), acc);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < DMAX; ++c)
          if (c < D) acc = fmaf(qr[c], to_f32(r[c]), acc);
      }
      return acc;
    };
    // each thread forms runs of 4 consecutive outputs and stores them together
    // (one 16-byte store when the row allows it)
    auto run = [&](float* out, int n, const TIN* tab, int tbase) {      // table row tbase - k for output k
      if (n < 4 * tpq) {           // few outputs per thread (small grids): one at a time, all threads busy
        for (int k = part; k < n; k += tpq) out[k] = dot(tab + (int64_t)(tbase - k) * pitch);
        return;
      }
      const bool v4 = (n & 3) == 0;
      for (int k0 = 4 * part; k0 < n; k0 += 4 * tpq) {
        float r4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r4[u] = (k0 + u < n) ? dot(tab + (int64_t)(tbase - k0 - u) * pitch) : 0.0f;
        if (v4) {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          *(f32x4*)(out + k0) = (f32x4){r4[0], r4[1], r4[2], r4[3]};
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (k0 + u < n) out[k0 + u] = r4[u];
        }
      }
    };
    run(p.term_h + (base + t) * gh, gh, rh, (int)row + gh - 1);
    run(p.term_w + (base + t) * gw, gw, rw, t + gw - 1);
    (void)pitch;
  }
}

template <typename TIN, int DMAX>
static void launch_terms_dim(const TermsParams& p, dim3 grid, hipStream_t s) {
  const bool vec = (p.D * (int64_t)sizeof(TIN)) % 16 == 0 && (((uintptr_t)p.rel_h | (uintptr_t)p.rel_w) & 15) == 0;
  const size_t lds = (size_t)(p.grid_h + 2 * p.grid_w - 1) * (p.D + 16 / sizeof(TIN)) * sizeof(TIN);
  if (vec && lds <= 64 * 1024)
    hipLaunchKernelGGL((relpos_terms_kernel<TIN, DMAX, true, true>), grid, dim3(256), lds, s, p);
  else if (vec)
    hipLaunchKernelGGL((relpos_terms_kernel<TIN, DMAX, true, false>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((relpos_terms_kernel<TIN, DMAX, false, false>), grid, dim3(256), 0, s, p);
}

template <typename TIN>
static void launch_terms_typed(const TermsParams& p, dim3 grid, hipStream_t s) {
  if (p.D <= 32) launch_terms_dim<TIN, 32>(p, grid, s);
  else if (p.D <= 64) launch_terms_dim<TIN, 64>(p, grid, s);
  else launch_terms_dim<TIN, 128>(p, grid, s);
}

hipError_t launch_relpos_terms(const TermsParams& p, hipStream_t s) {
  dim3 grid((unsigned)p.grid_h, (unsigned)p.H, (unsigned)p.B);
  if (p.dtype == 0) launch_terms_typed<float>(p, grid, s);
  else if (p.dtype == 2) launch_terms_typed<_Float16>(p, grid, s);
  else launch_terms_typed<__bf16>(p, grid, s);
  return hipGetLastError();
}

}  // namespace sdpa
