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
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// ------------------------------------------- table gradients on MFMA ------
// Both tables' gradients as products on the matrix cores (fp32 operands, the
// 32x32x2 fp32 matrix op, so dT enters unrounded).  The queries are taken by
// lines: grid rows r for rel_pos_h (the line's grid_w queries share row(i) =
// r), grid columns c for rel_pos_w (grid_h queries, col(i) = c).  For a table
// of width G (G = grid_h for rows, grid_w for columns) and a line l, entry t
// of the gradient collects dT[i][a] q_i over the line's queries with
// a = l + G - 1 - t:
//   dR[t][d] += sum_i A_l[t][i] q_i[d],   A_l[t][i] = dT[i][l + G - 1 - t]  (0 outside [0, G)).
// A workgroup takes a run of (batch, head, line) items of one table
// (blockIdx.y: 0 rows, 1 columns) and keeps the [2G - 1 <= 127 rows x D] sums
// in MFMA accumulators, wave w owning rows 32w .. 32w + 31 (a wave whose rows
// the line does not reach skips it); each workgroup's sums go to scratch and
// a second kernel adds them in a fixed order (deterministic, no atomics).
constexpr int kTgPad = 32;                     // row padding (floats): the two query rows of an MFMA k pair hit other banks
constexpr int kTgGP = 64 + kTgPad;             // dT row stride in LDS (a 64-lane copy fills the first 64 floats)
constexpr int kDqGP = 65;                      // the dq kernel's dT row stride: odd, >= 64

// LDS bytes of one staging buffer: dT rows [L][kTgGP] fp32 and q rows [L rounded
// up to 4][D] in the input type (a q copy moves up to 4 rows at once).
__host__ __device__ inline int tg_buf_bytes(int L, int D) { return L * kTgGP * 4 + (L + 3) / 4 * 4 * D * 2; }

template <typename E, int D>
__global__ __launch_bounds__(256) void relpos_tgrad_kernel(BwdParams p, int ipw_h, int ipw_w) {
  constexpr int DB = D / 32;
  constexpr int QRB = D * 2;                    // bytes of one q row
  constexpr int QRPI = 256 / QRB;               // q rows one 64-lane 4-byte copy moves (D 32: 4, 64: 2, 128: 1)
  extern __shared__ __attribute__((aligned(16))) char tg_lds[];   // two staging buffers
  const bool rows = blockIdx.y == 0;
  const int gh = p.grid_h, gw = p.grid_w;
  const int G = rows ? gh : gw, L = rows ? gw : gh;
  const int BUF = tg_buf_bytes(L, D);
  const float* dT = rows ? p.dterm_h : p.dterm_w;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int trow = 32 * wave + (lane & 31), kh = lane >> 5;
  const int64_t T = p.Tq;
  // Descriptors over all of dT and q: a lane past its row's end reads the next
  // row (it lands in LDS padding) or, past the array, 0.
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)dT, 0, (int)(p.B * p.Hq * T * G * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.q, 0, (int)(((p.B - 1) * p.q_sb + (p.Hq - 1) * p.q_sh + (T - 1) * p.q_st + D) * 2), 0x00020000);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  const int64_t items = p.B * p.Hq * G;
  const int ipw = rows ? ipw_h : ipw_w;
  const int64_t it0 = (int64_t)blockIdx.x * ipw, it1 = min(items, it0 + ipw);
  const int64_t istep = rows ? 1 : gw;          // query index step along the line
  // Copies of a line's rows straight into LDS buffer `buf` (no registers):
  // dT row qi -> 64 floats at row qi of the dT region; q rows in groups of QRPI.
  auto issue = [&](int64_t it, int buf) {
    const int64_t bh = it / G;
    const int line = (int)(it - bh * G);
    const int bh32 = (int)bh, hq32 = (int)p.Hq;        // B * Hq < 2^16
    const int64_t b = bh32 / hq32, h = bh32 - (bh32 / hq32) * hq32;
    const int64_t ibase = rows ? (int64_t)line * gw : (int64_t)line;
    char* base = tg_lds + buf * BUF;
    for (int qi = wave; qi < L; qi += 4) {
      const int64_t i = ibase + qi * istep;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(base + qi * kTgGP * 4), 4,
                                               (int)(((bh * T + i) * G + lane) * 4), 0, 0, 0);
    }
    char* qbase = base + L * kTgGP * 4;
    for (int q0 = wave * QRPI; q0 < L; q0 += 4 * QRPI) {
      const int qi = q0 + lane / (64 / QRPI);
      const int64_t i = ibase + (qi < L ? qi : q0) * istep;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qrs, (__attribute__((address_space(3))) void*)(qbase + q0 * QRB), 4,
          (int)((b * p.q_sb + h * p.q_sh + i * p.q_st) * 2 + (lane % (64 / QRPI)) * 4), 0, 0, 0);
    }
  };
  if (it0 < it1) issue(it0, 0);
  for (int64_t it = it0; it < it1; ++it) {
    const int buf = (int)((it - it0) & 1);
    const int line = (int)(it - (it / G) * G);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                                   // this line's rows landed; the other buffer is free
    if (it + 1 < it1) issue(it + 1, buf ^ 1);
    if (32 * wave > line + G - 1 || 32 * wave + 31 < line) continue;   // rows this line does not reach
    const float* dts = (const float*)(tg_lds + buf * BUF);
    const E* qs = (const E*)(tg_lds + buf * BUF + L * kTgGP * 4);
    const int a = line + G - 1 - trow;
    const bool aok = a >= 0 && a < G;
    const float* ar = dts + (aok ? a : 0) + kh * kTgGP;
    const E* br = qs + (lane & 31) + kh * D;
    int k0 = 0;
    // 8 k pairs (16 queries) at a time: every LDS read of the batch is issued
    // before its matrix ops
    for (; k0 + 16 <= L; k0 += 16) {
      float av[8], bv[8][DB];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[j] = aok ? ar[(k0 + 2 * j) * kTgGP] : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) bv[j][db] = (float)br[(k0 + 2 * j) * D + 32 * db];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j][db], acc[db], 0, 0, 0);
    }
    for (; k0 < L; k0 += 2) {
      const bool qok = k0 + kh < L;
      const float av = (aok && qok) ? ar[k0 * kTgGP] : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const float bv = qok ? (float)br[k0 * D + 32 * db] : 0.0f;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[db], 0, 0, 0);
      }
    }
  }
  // this workgroup's sums: [128 rows t][D], rows 8 (r / 4) + 4 kh + r % 4 of the wave's block
  float* out = (rows ? p.group_h : p.group_w) + (int64_t)blockIdx.x * 128 * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      out[(32 * wave + 8 * (r / 4) + 4 * kh + (r % 4)) * D + 32 * db + (lane & 31)] = acc[db][r];
}

// Small grids (both sides <= 16: SAM's 14 x 14 windows): the 2G - 1 <= 31
// gradient rows fit one 32-row block, so each wave takes its own run of lines
// with its own staging buffers and keeps all of them in its accumulators;
// the four waves' sums are added in LDS, and the workgroup writes rows
// 0 .. 31 of its partial.  A line's <= 16 dT rows of
// <= 16 floats go to LDS four rows per 64-lane copy, its q rows one to four
// per copy.
constexpr int kTsRows = 16;                    // line length and table width the small mode takes
__host__ __device__ inline int ts_buf_bytes(int D) { return kTsRows * 16 * 4 + kTsRows * D * 2; }

template <typename E, int D>
__global__ __launch_bounds__(256) void relpos_tgrad_small_kernel(BwdParams p, int ipw_h, int ipw_w) {
  constexpr int DB = D / 32;
  constexpr int QRB = D * 2;
  constexpr int QRPI = 256 / QRB;
  extern __shared__ __attribute__((aligned(16))) char ts_lds[];   // [wave][2 buffers]
  const bool rows = blockIdx.y == 0;
  const int gh = p.grid_h, gw = p.grid_w;
  const int G = rows ? gh : gw, L = rows ? gw : gh;
  const float* dT = rows ? p.dterm_h : p.dterm_w;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int trow = lane & 31, kh = lane >> 5;
  const int64_t T = p.Tq;
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)dT, 0, (int)(p.B * p.Hq * T * G * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.q, 0, (int)(((p.B - 1) * p.q_sb + (p.Hq - 1) * p.q_sh + (T - 1) * p.q_st + D) * 2), 0x00020000);
  char* mine = ts_lds + wave * 2 * ts_buf_bytes(D);
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = (f32x16){};
  const int64_t items = p.B * p.Hq * G;
  const int ipw = rows ? ipw_h : ipw_w;
  const int64_t wid = (int64_t)blockIdx.x * 4 + wave;
  const int64_t it0 = wid * ipw, it1 = min(items, it0 + ipw);
  const int64_t istep = rows ? 1 : gw;
  auto issue = [&](int64_t it, int buf) {
    const int64_t bh = it / G;
    const int line = (int)(it - bh * G);
    const int bh32 = (int)bh, hq32 = (int)p.Hq;        // B * Hq < 2^16
    const int64_t b = bh32 / hq32, h = bh32 - (bh32 / hq32) * hq32;
    const int64_t ibase = rows ? (int64_t)line * gw : (int64_t)line;
    char* base = mine + buf * ts_buf_bytes(D);
    // dT rows: lane l -> row 4 c + l / 16, column l % 16 (rows and columns past L, G land in padding)
#pragma unroll
    for (int c = 0; c < kTsRows / 4; ++c) {
      const int qi = 4 * c + lane / 16;
      const int64_t i = ibase + (qi < L ? qi : 0) * istep;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(base + c * 256), 4,
                                               (int)(((bh * T + i) * G + (lane % 16)) * 4), 0, 0, 0);
    }
    char* qbase = base + kTsRows * 16 * 4;
#pragma unroll
    for (int q0 = 0; q0 < kTsRows; q0 += QRPI) {
      const int qi = q0 + lane / (64 / QRPI);
      const int64_t i = ibase + (qi < L ? qi : 0) * istep;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qrs, (__attribute__((address_space(3))) void*)(qbase + q0 * QRB), 4,
          (int)((b * p.q_sb + h * p.q_sh + i * p.q_st) * 2 + (lane % (64 / QRPI)) * 4), 0, 0, 0);
    }
  };
  if (it0 < it1) issue(it0, 0);
  for (int64_t it = it0; it < it1; ++it) {
    const int buf = (int)((it - it0) & 1);
    const int line = (int)(it - (it / G) * G);
    __builtin_amdgcn_s_waitcnt(0);                    // this line's rows are in LDS (copies of this wave only)
    wave_sync();                                      // and the wave's reads of the other buffer are done
    if (it + 1 < it1) issue(it + 1, buf ^ 1);
    const float* dts = (const float*)(mine + buf * ts_buf_bytes(D));
    const E* qs = (const E*)(mine + buf * ts_buf_bytes(D) + kTsRows * 16 * 4);
    const int a = line + G - 1 - trow;
    const bool aok = a >= 0 && a < G;
    const float* ar = dts + (aok ? a : 0) + kh * 16;
    const E* br = qs + (lane & 31) + kh * D;
    for (int k0 = 0; k0 < L; k0 += 2) {
      const bool qok = k0 + kh < L;
      const float av = (aok && qok) ? ar[k0 * 16] : 0.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const float bv = qok ? (float)br[k0 * D + 32 * db] : 0.0f;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[db], 0, 0, 0);
      }
    }
    wave_sync();                                      // reads of this buffer done before the next issue
  }
  // the four waves' sums meet in LDS ([wave][32 rows][D]) and add in wave
  // order (fixed); the workgroup's partial is rows 0 .. 31 of its 128-row slot
  __syncthreads();                                    // every wave is done with its staging buffers
  float* red = (float*)ts_lds;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      red[(wave * 32 + 8 * (r / 4) + 4 * kh + (r % 4)) * D + 32 * db + (lane & 31)] = acc[db][r];
  __syncthreads();
  float* out = (rows ? p.group_h : p.group_w) + (int64_t)blockIdx.x * 128 * D;
  for (int e = tid; e < 32 * D; e += 256)
    out[e] = ((red[e] + red[32 * D + e]) + red[2 * 32 * D + e]) + red[3 * 32 * D + e];
}

// dR[t][d] = sum over the nwg workgroups' partial sums: thread (g, d) of a
// workgroup adds the partials w = g, g + 4, ... of entry (t, d) for 64 head
// dims (a wave reads 256 contiguous bytes of one partial row), then the four
// sums add in order: a fixed order.  Grid: (max(2 grid_h - 1, 2 grid_w - 1),
// ceil(D / 64), 2 tables).
__global__ __launch_bounds__(256) void relpos_tgrad_reduce_kernel(BwdParams p, int nwg, int D) {
  __shared__ float red[4][64];
  const bool rows = blockIdx.z == 0;
  const int Tn = 2 * (rows ? p.grid_h : p.grid_w) - 1;
  const int t = blockIdx.x;
  if (t >= Tn) return;                                // the whole workgroup
  const float* part = rows ? p.group_h : p.group_w;
  const int g = threadIdx.x >> 6, dd = threadIdx.x & 63, d = blockIdx.y * 64 + dd;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (d < D) {
    int w = g;
    for (; w + 28 < nwg; w += 32) {                    // eight loads in flight, into four sums
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[((int64_t)(w + 4 * u) * 128 + t) * D + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u & 3] += v[u];
    }
    for (; w < nwg; w += 4) acc[0] += part[((int64_t)w * 128 + t) * D + d];
  }
  red[g][dd] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (g == 0 && d < D)
    (rows ? p.drel_h : p.drel_w)[(int64_t)t * D + d] = ((red[0][dd] + red[1][dd]) + red[2][dd]) + red[3][dd];
}

// ---------------------------------------------- tables' part of dq, MFMA --
// dq_i = dQ_acc_i + sum_y dT_h[i, y] Rh[row(i) - y + gh - 1] + sum_x dT_w[i, x] Rw[col(i) - x + gw - 1]
// as line products on the matrix cores (fp32 operands): for a grid row r the
// term_h part of its queries c is [c][y] x [y][d] with the reversed table
// rows Rh[r + gh - 1 - y]; for a grid column c the term_w part of its
// queries likewise with Rw[c + gw - 1 - x].  Pass ROWS adds the term_h part
// into the fp32 dQ_acc; pass !ROWS adds the term_w part and writes dq.  One
// workgroup per (batch, head, line); wave w owns output blocks w and w + 4 of
// the [L (<= 64) queries x D] result (32 x 32 blocks, query blocks outer).
// LDS bytes of one line: dT rows [L][kDqGP] fp32 and table rows [G rounded up to 4][D].
__host__ __device__ inline int dq_lds_bytes(int L, int G, int D) { return L * kDqGP * 4 + (G + 3) / 4 * 4 * D * 2; }

template <typename E, int D, typename GT, bool ROWS>
__global__ __launch_bounds__(256) void relpos_dq_mfma_kernel(BwdParams p) {
  constexpr int DB = D / 32;
  constexpr int QRB = D * 2;                    // bytes of one table row
  constexpr int QRPI = 256 / QRB;               // table rows one 64-lane 4-byte copy moves
  extern __shared__ __attribute__((aligned(16))) char dq_lds[];
  const int gh = p.grid_h, gw = p.grid_w;
  const int G = ROWS ? gh : gw, L = ROWS ? gw : gh;
  const int MB = (L + 31) / 32;
  // Lines with fewer than four 32 x 32 output blocks share a workgroup: ipg
  // lines, wpi = 4 / ipg waves each (wave sub-index wv).
  const int nblk = MB * DB, ipg = nblk >= 4 ? 1 : 4 / nblk, wpi = 4 / ipg;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = wave / wpi, wv = wave - sub * wpi;
  const int64_t item = (int64_t)blockIdx.x * ipg + sub;
  const bool have = item < p.B * p.Hq * G;
  // Per line: dT rows of its queries [L][kDqGP] fp32 (odd stride: the 32 query
  // rows of an A read hit 32 banks), then the reversed table rows
  // tab[a] = R[line + G - 1 - a], [G rounded up to 4][D] in the input type.
  char* region = dq_lds + sub * dq_lds_bytes(L, G, D);
  const float* dts = (const float*)region;
  const E* tab = (const E*)(region + L * kDqGP * 4);
  const float* dT = ROWS ? p.dterm_h : p.dterm_w;
  const E* R = (const E*)(ROWS ? p.rel_h : p.rel_w);
  const int kh = lane >> 5, l32 = lane & 31;
  const int64_t bh = have ? item / G : 0;
  const int line = (int)(have ? item - bh * G : 0);
  const int bh32 = (int)bh, hq32 = (int)p.Hq;           // B * Hq < 2^16
  const int64_t b = bh32 / hq32, h = bh32 - (bh32 / hq32) * hq32;
  const int64_t T = p.Tq;
  auto query = [&](int qi) -> int64_t { return ROWS ? (int64_t)line * gw + qi : (int64_t)qi * gw + line; };
  // Copies straight into LDS (no registers, one memory round trip): a lane
  // past its row's end reads the next row (LDS padding) or, past the array, 0.
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)dT, 0, (int)(p.B * p.Hq * T * G * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)R, 0, (int)((2 * G - 1) * D * 2), 0x00020000);
  for (int qi = have ? wv : L; qi < L; qi += wpi)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(region + qi * kDqGP * 4), 4,
                                             (int)(((bh * T + query(qi)) * G + lane) * 4), 0, 0, 0);
  char* tbase = region + L * kDqGP * 4;
  for (int a0 = have ? wv * QRPI : G; a0 < G; a0 += wpi * QRPI) {
    const int a = a0 + lane / (64 / QRPI);
    const int ra = line + G - 1 - (a < G ? a : a0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rrs, (__attribute__((address_space(3))) void*)(tbase + a0 * QRB), 4,
                                             (int)(ra * QRB + (lane % (64 / QRPI)) * 4), 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // this lane's dQ_acc entries of its (at most two) output blocks, requested
  // now so that their round trip passes under the products
  float pre[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int blk = wv + wpi * u;
    const int mb = blk / DB, db = blk - mb * DB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 32 * mb + 8 * (r / 4) + 4 * kh + (r % 4);
      pre[u][r] = (have && blk < nblk && qi < L) ? p.dq_acc[(bh * T + query(qi)) * D + 32 * db + l32] : 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int blk = wv + wpi * u;
    if (!have || blk >= nblk) break;
    const int mb = blk / DB, db = blk - mb * DB;
    const int qrow = 32 * mb + l32;
    const bool qok = qrow < L;
    const float* ar = dts + (qok ? qrow : 0) * kDqGP + kh;
    const E* br = tab + kh * D + 32 * db + l32;
    f32x16 acc = (f32x16){};
    int k0 = 0;
    for (; k0 + 16 <= G; k0 += 16) {
      float av[8], bv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[j] = qok ? ar[k0 + 2 * j] : 0.0f;
        bv[j] = (float)br[(k0 + 2 * j) * D];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
    }
    for (; k0 < G; k0 += 2) {
      const bool kok = k0 + kh < G;
      const float av = (qok && kok) ? ar[k0] : 0.0f;
      const float bv = kok ? (float)br[k0 * D] : 0.0f;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    // rows 8 (r / 4) + 4 kh + r % 4 of the block are queries, the lane's column a head dim
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 32 * mb + 8 * (r / 4) + 4 * kh + (r % 4);
      if (qi >= L) continue;
      const int64_t i = query(qi);
      const int d = 32 * db + l32;
      if (ROWS) p.dq_acc[(bh * T + i) * D + d] = pre[u][r] + acc[r];
      else ((GT*)p.dq)[b * p.q_sb + h * p.q_sh + i * p.q_st + d] = (GT)(pre[u][r] + acc[r]);
    }
  }
}

template <int D>
bool relpos_dq_mfma_ok(const BwdParams& p) {
  const int64_t gh = p.grid_h, gw = p.grid_w;
  // dT through a descriptor with 32-bit byte offsets; LDS: dT rows plus table rows
  return gh <= 64 && gw <= 64 && p.B * p.Hq * gh * gw * (gh > gw ? gh : gw) * 4 <= 0x7fffffffLL;
}

// The tables' gradients d rel_pos_h / d rel_pos_w from dterm_h / dterm_w and q.
template <typename E, int D>
void tables_typed(const BwdParams& p, hipStream_t s) {
  if (relpos_tgrad_mfma_ok(p.B, p.Hq, p.grid_h, p.grid_w, D) && p.tgrad_mfma) {
    const int nwg = relpos_tgrad_wgs(p.B, p.Hq, p.grid_h, p.grid_w);
    const int64_t ih = p.B * p.Hq * p.grid_h, iw = p.B * p.Hq * p.grid_w;
    const int tmax = 2 * (p.grid_h > p.grid_w ? p.grid_h : p.grid_w) - 1;
    if (p.grid_h <= kTsRows && p.grid_w <= kTsRows) {
      const int nw = 4 * nwg;                         // waves, each with its own run of lines
      const size_t lds = std::max((size_t)(4 * 2 * ts_buf_bytes(D)), (size_t)(4 * 32 * D * 4));
      hipLaunchKernelGGL((relpos_tgrad_small_kernel<E, D>), dim3((unsigned)nwg, 2u), dim3(256), lds, s, p,
                         (int)((ih + nw - 1) / nw), (int)((iw + nw - 1) / nw));
      hipLaunchKernelGGL(relpos_tgrad_reduce_kernel, dim3((unsigned)tmax, (unsigned)((D + 63) / 64), 2u), dim3(256),
                         0, s, p, nwg, D);
      return;
    }
    const size_t lds = 2 * (size_t)std::max(tg_buf_bytes(p.grid_w, D), tg_buf_bytes(p.grid_h, D));
    hipLaunchKernelGGL((relpos_tgrad_kernel<E, D>), dim3((unsigned)nwg, 2u), dim3(256), lds, s, p,
                       (int)((ih + nwg - 1) / nwg), (int)((iw + nwg - 1) / nwg));
    hipLaunchKernelGGL(relpos_tgrad_reduce_kernel, dim3((unsigned)tmax, (unsigned)((D + 63) / 64), 2u), dim3(256), 0,
                       s, p, nwg, D);
    return;
  }
  hipLaunchKernelGGL((relpos_group_kernel<E, D, true>), dim3((unsigned)p.grid_h, (unsigned)p.split_h), dim3(256), 0, s, p);
  hipLaunchKernelGGL((relpos_group_kernel<E, D, false>), dim3((unsigned)p.grid_w, (unsigned)p.split_w), dim3(256), 0, s, p);
  hipLaunchKernelGGL(relpos_diag_kernel, dim3((unsigned)((D + 15) / 16), (unsigned)(2 * p.grid_h - 1)), dim3(256), 0, s,
                     (const float*)p.group_h, p.drel_h, p.grid_h, D, p.split_h);
  hipLaunchKernelGGL(relpos_diag_kernel, dim3((unsigned)((D + 15) / 16), (unsigned)(2 * p.grid_w - 1)), dim3(256), 0, s,
                     (const float*)p.group_w, p.drel_w, p.grid_w, D, p.split_w);
}

template <typename E, int D, typename G>
void tail_typed(const BwdParams& p, hipStream_t s, bool dq_part) {
  if (!dq_part) {
    tables_typed<E, D>(p, s);
    return;
  }
  if (p.tgrad_mfma && relpos_dq_mfma_ok<D>(p)) {
    // lines per workgroup as the kernel derives them: 4 / (32 x 32 output blocks per line), at least 1
    auto ipg = [](int L) { const int nb = (L + 31) / 32 * (D / 32); return nb >= 4 ? 1 : 4 / nb; };
    const int ih = ipg(p.grid_w), iw = ipg(p.grid_h);
    const int64_t nh = p.B * p.Hq * p.grid_h, nw = p.B * p.Hq * p.grid_w;
    hipLaunchKernelGGL((relpos_dq_mfma_kernel<E, D, G, true>), dim3((unsigned)((nh + ih - 1) / ih)), dim3(256),
                       (size_t)ih * dq_lds_bytes(p.grid_w, p.grid_h, D), s, p);
    hipLaunchKernelGGL((relpos_dq_mfma_kernel<E, D, G, false>), dim3((unsigned)((nw + iw - 1) / iw)), dim3(256),
                       (size_t)iw * dq_lds_bytes(p.grid_h, p.grid_w, D), s, p);
  } else {
    constexpr int QPB = 256 / (D / 16);
    dim3 gq((unsigned)((p.Tq + QPB - 1) / QPB), (unsigned)(p.B * p.Hq));
    hipLaunchKernelGGL((relpos_bwd_dq_kernel<E, D, G>), gq, dim3(256), 0, s, p);
  }
}

template <typename E, int D>
void tail_g(const BwdParams& p, hipStream_t s, bool dq_part) {
  if (p.grad_dtype == 0) tail_typed<E, D, float>(p, s, dq_part);
  else tail_typed<E, D, E>(p, s, dq_part);
}

template <typename E>
void tail_e(const BwdParams& p, hipStream_t s, bool dq_part) {
  if (p.D == 32) tail_g<E, 32>(p, s, dq_part);
  else if (p.D == 64) tail_g<E, 64>(p, s, dq_part);
  else tail_g<E, 128>(p, s, dq_part);
}

}  // namespace

hipError_t launch_relpos_bwd_dq(const BwdParams& p, hipStream_t s) {
  if (p.dtype == 2) tail_e<_Float16>(p, s, true);
  else tail_e<__bf16>(p, s, true);
  return hipGetLastError();
}

hipError_t launch_relpos_bwd_tables(const BwdParams& p, hipStream_t s) {
  if (p.dtype == 2) tail_e<_Float16>(p, s, false);
  else tail_e<__bf16>(p, s, false);
  return hipGetLastError();
}

}  // namespace sdpa
