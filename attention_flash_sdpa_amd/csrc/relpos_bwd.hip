// Rel-pos tail of the attention backward pass.
//
// SAM's decomposed bias ([mlx-examples issue 1451] "segment_anything: fuse
// attention with mx.fast.scaled_dot_product_attention", body:
// add_decomposed_rel_pos; [Candle PR 3280] "feat(metal): SDPA with Relative
// Positional Embeddings & LayerNorm Stability", Key Changes: term_h / term_w)
// is B[i, j] = term_h[i, row(j)] + term_w[i, col(j)] with
//   term_h[i, y] = q_i . Rh[row(i) - y + gh - 1],  term_w[i, x] = q_i . Rw[col(i) - x + gw - 1].
// The attention kernels leave dT_h[i, y] = sum of dS[i, j] over the keys j of
// grid row y (dT_w over grid column x) and dQ_acc = scale * dS . K.  Here:
//   dq_i   = dQ_acc_i + sum_y dT_h[i, y] Rh[row(i) - y + gh - 1] + sum_x dT_w[i, x] Rw[col(i) - x + gw - 1]
//   dRh[t] = sum over (b, h, i, y) with row(i) - y + gh - 1 = t of dT_h[i, y] q_i    (dRw alike).
// The table gradients are grouped by the query's grid row r (columns c for
// Rw): G_h[r][y] = sum over (b, h) and the gw queries of row r of dT_h[i, y] q_i
// (a [gh x D] product per row, cut into slices of the queries so that several
// hundred workgroups share the work), then dRh[t] = sum over slices and rows r
// of G_h[r][r + gh - 1 - t], a fixed-order sum (no atomics: the result is
// deterministic).
#include "common.h"

namespace sdpa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTabRows = 2 * 128 - 2;     // (2 gh - 1) + (2 gw - 1) with gh + gw <= 128

// --------------------------------------------------------------- dq ------
template <typename E, int D, typename G>
__global__ __launch_bounds__(256) void relpos_bwd_dq_kernel(BwdParams p) {
  constexpr int TPQ = D / 16;            // threads per query, 16 head dims each
  constexpr int QPB = 256 / TPQ;         // queries per workgroup
  // [Rh rows | Rw rows][D + 4] fp32: the 4-float pad shifts consecutive rows by
  // 16 bytes of banks, so the 16 queries a wave reads (different rows) spread out
  constexpr int TP = D + 4;
  __shared__ __attribute__((aligned(16))) float tab[kMaxTabRows * TP];
  const int gh = p.grid_h, gw = p.grid_w, nh = 2 * gh - 1, nw = 2 * gw - 1;
  const int tid = threadIdx.x;
  const E* rh = (const E*)p.rel_h;
  const E* rw = (const E*)p.rel_w;
  for (int e = tid; e < (nh + nw) * D; e += 256) {
    const int t = e / D, c = e % D;
    tab[t * TP + c] = (float)(e < nh * D ? rh[e] : rw[e - nh * D]);
  }
  __syncthreads();
  const int64_t bh = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * QPB + tid / TPQ;
  if (i >= p.Tq) return;
  const int d0 = (tid % TPQ) * 16;
  const int64_t srow = bh * p.Tq + i;
  const int row = (int)(i / gw), col = (int)(i % gw);
  float acc[16];
  const float* qa = p.dq_acc + srow * D + d0;
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const f32x4 v = *(const f32x4*)(qa + e);
    acc[e] = v[0]; acc[e + 1] = v[1]; acc[e + 2] = v[2]; acc[e + 3] = v[3];
  }
  const float* th = p.dterm_h + srow * gh;
#pragma unroll 4
  for (int y = 0; y < gh; ++y) {
    const float c = th[y];
    const float* t = tab + (row - y + gh - 1) * TP + d0;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(c, t[e], acc[e]);
  }
  const float* tw = p.dterm_w + srow * gw;
#pragma unroll 4
  for (int x = 0; x < gw; ++x) {
    const float c = tw[x];
    const float* t = tab + (nh + col - x + gw - 1) * TP + d0;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(c, t[e], acc[e]);
  }
  const int64_t b = bh / p.Hq, h = bh % p.Hq;
  G* out = (G*)p.dq + b * p.q_sb + h * p.q_sh + i * p.q_st + d0;
#pragma unroll
  for (int e = 0; e < 16; ++e) out[e] = (G)acc[e];
}

// ------------------------------------------------------ grouped products --
// out[gidx][a][d] = sum over (b, h) and the members i of group gidx of A[b, h, i][a] * q[b, h, i][d].
// ROWS: groups are grid rows (members r * gw + x), else grid columns (members y * gw + c).
template <typename E, int D, bool ROWS>
__global__ __launch_bounds__(256) void relpos_group_kernel(BwdParams p) {
  constexpr int CM = 16;                  // members staged per step
  __shared__ float as[CM][64 + 1];
  __shared__ float qs[CM][64 + 1];
  const int gh = p.grid_h, gw = p.grid_w;
  const int aw = ROWS ? gh : gw;          // width of A (entries per query)
  const int nmem = ROWS ? gw : gh;        // members per (b, h)
  const float* A = ROWS ? p.dterm_h : p.dterm_w;
  const int ngroups = ROWS ? gh : gw;
  const int gidx = blockIdx.x;
  // this workgroup's slice of the group's members (queries over every (b, h))
  const int64_t total = p.B * p.Hq * nmem;
  const int nsplit = gridDim.y;
  const int64_t per = ((total + nsplit - 1) / nsplit + CM - 1) / CM * CM;
  const int64_t m_lo = (int64_t)blockIdx.y * per, m_hi = min(total, m_lo + per);
  float* out = (ROWS ? p.group_h : p.group_w) + ((int64_t)blockIdx.y * ngroups + gidx) * aw * D;
  const int tid = threadIdx.x, ta = tid / 16, td = tid % 16;
  // Staging: thread tid fills column c = tid % 64 of members m = tid / 64 + 4 u (u = 0..3)
  // of each 16-member step; each slot's member index advances by 16 per step, so its
  // (b, h, k) position is stepped forward instead of divided out per element.
  const int c = tid % 64;
  int64_t bh0[4];
  int k0[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t mm = m_lo + tid / 64 + 4 * u;
    bh0[u] = mm / nmem;
    k0[u] = (int)(mm % nmem);
  }
  for (int oa = 0; oa < aw; oa += 64)
    for (int od = 0; od < D; od += 64) {
      float acc[4][4] = {};
      int64_t bh[4];
      int kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bh[u] = bh0[u];
        kk[u] = k0[u];
      }
      for (int64_t m0 = m_lo; m0 < m_hi; m0 += CM) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = tid / 64 + 4 * u;
          float av = 0.0f, qv = 0.0f;
          if (m0 + m < m_hi) {
            const int64_t i = ROWS ? (int64_t)gidx * gw + kk[u] : (int64_t)kk[u] * gw + gidx;
            if (oa + c < aw) av = A[(bh[u] * p.Tq + i) * aw + oa + c];
            if (od + c < D) {
              const int bh32 = (int)bh[u], hq32 = (int)p.Hq;    // B * Hq < 2^16
              const int64_t b = bh32 / hq32, h = bh32 - (bh32 / hq32) * hq32;
              qv = (float)((const E*)p.q)[b * p.q_sb + h * p.q_sh + i * p.q_st + od + c];
            }
          }
          as[m][c] = av;
          qs[m][c] = qv;
          kk[u] += CM;                       // the slot's next member: 16 further on
          while (kk[u] >= nmem) {
            kk[u] -= nmem;
            ++bh[u];
          }
        }
        __syncthreads();
#pragma unroll 4
        for (int m = 0; m < CM; ++m) {
          float a4[4], q4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            a4[u] = as[m][4 * ta + u];
            q4[u] = qs[m][4 * td + u];
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a4[u], q4[v], acc[u][v]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int a = oa + 4 * ta + u, d = od + 4 * td + v;
          if (a < aw && d < D) out[a * D + d] = acc[u][v];
        }
    }
}

// dR[t][d] = sum over slices s and groups r of G[s][r][r + n - 1 - t][d], for the
// entries with 0 <= r + n - 1 - t < n.  One workgroup per (16 head dims, t): 16
// partial sums per dim over the (s, r) pairs k = s * n + r with k % 16 = part,
// then added in part order (a fixed order: deterministic).
__global__ __launch_bounds__(256) void relpos_diag_kernel(const float* G, float* dR, int n, int D, int nsplit) {
  __shared__ float red[16][16];
  const int part = threadIdx.x / 16, dd = threadIdx.x % 16;
  const int d = blockIdx.x * 16 + dd, t = blockIdx.y;
  float acc = 0.0f;
  if (d < D) {
    for (int k = part; k < nsplit * n; k += 16) {
      const int sl = k / n, r = k % n, y = r + n - 1 - t;
      if (y >= 0 && y < n) acc += G[(((int64_t)sl * n + r) * n + y) * D + d];
    }
  }
  red[part][dd] = acc;
  __syncthreads();
  if (part == 0 && d < D) {
    float tot = 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) tot += red[u][dd];
    dR[(int64_t)t * D + d] = tot;
  }
}

template <typename E, int D, typename G>
void tail_typed(const BwdParams& p, hipStream_t s) {
  constexpr int QPB = 256 / (D / 16);
  dim3 gq((unsigned)((p.Tq + QPB - 1) / QPB), (unsigned)(p.B * p.Hq));
  hipLaunchKernelGGL((relpos_bwd_dq_kernel<E, D, G>), gq, dim3(256), 0, s, p);
  hipLaunchKernelGGL((relpos_group_kernel<E, D, true>), dim3((unsigned)p.grid_h, (unsigned)p.split_h), dim3(256), 0, s, p);
  hipLaunchKernelGGL((relpos_group_kernel<E, D, false>), dim3((unsigned)p.grid_w, (unsigned)p.split_w), dim3(256), 0, s, p);
  hipLaunchKernelGGL(relpos_diag_kernel, dim3((unsigned)((D + 15) / 16), (unsigned)(2 * p.grid_h - 1)), dim3(256), 0, s,
                     (const float*)p.group_h, p.drel_h, p.grid_h, D, p.split_h);
  hipLaunchKernelGGL(relpos_diag_kernel, dim3((unsigned)((D + 15) / 16), (unsigned)(2 * p.grid_w - 1)), dim3(256), 0, s,
                     (const float*)p.group_w, p.drel_w, p.grid_w, D, p.split_w);
}

template <typename E, int D>
void tail_g(const BwdParams& p, hipStream_t s) {
  if (p.grad_dtype == 0) tail_typed<E, D, float>(p, s);
  else tail_typed<E, D, E>(p, s);
}

template <typename E>
void tail_e(const BwdParams& p, hipStream_t s) {
  if (p.D == 32) tail_g<E, 32>(p, s);
  else if (p.D == 64) tail_g<E, 64>(p, s);
  else tail_g<E, 128>(p, s);
}

}  // namespace

hipError_t launch_relpos_bwd_tail(const BwdParams& p, hipStream_t s) {
  if (p.dtype == 2) tail_e<_Float16>(p, s);
  else tail_e<__bf16>(p, s);
  return hipGetLastError();
}

}  // namespace sdpa
