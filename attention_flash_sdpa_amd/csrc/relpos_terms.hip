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
//
// Two kernels.  16-bit inputs with head_dim 32, 64 or 128 on grids whose
// products fit a 32 x 128 slot (SAM's 14 x 14 windows and 64 x 64 global
// grid among them) run on the matrix cores: a wave takes 32 consecutive
// tokens, forms the products P[i, r] = q_i . table[r] for every table row r
// that any of its tokens needs (32 x 32 x 16 matrix ops, Q^T as the shared
// operand), stores them in its own LDS slot and then reads each token's term
// rows out of the slot along the skew r = coord(i) - y + G - 1.  The 32
// tokens' term rows are one contiguous stretch of each output array, written
// with 16-byte stores by consecutive lanes.  Other inputs use the vector-ALU
// kernel below.
#include "common.h"
#include "elem16.h"

namespace sdpa {

namespace {
constexpr int TRMAX = 128;            // table rows one 32-token block's products cover at most
constexpr int TPITCH = TRMAX + 4;     // slot pitch (floats): 16-byte aligned rows, consecutive tokens four banks apart
// Waves per workgroup of the matrix-core kernel.  The waves share nothing, so
// one-wave workgroups (17 KB of LDS each) let the dispatcher spread the waves
// evenly over the CUs: 1536 waves of SAM ViT-B global attention land 6 per CU
// instead of 4 or 8 in 384 workgroups of four.
constexpr int TWPB = 1;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Rows of the product one block needs: term_h spans grid rows row0..row1 of
// its tokens plus grid_h - 1; term_w spans columns col0..col1 plus grid_w - 1
// when the block lies in one grid row, else the whole table.
__host__ __device__ inline int terms_rows_h(int gh, int gw) { return gh + (gw + 30) / gw; }
__host__ __device__ inline int terms_rows_w(int gw) { return gw % 32 == 0 ? 31 + gw : 2 * gw - 1; }
}  // namespace

template <typename E, int NC>
__global__ __launch_bounds__(64 * TWPB) void relpos_terms_mfma_kernel(TermsParams p) {
  typedef typename Vec16<E>::x8 e8;
  __shared__ __attribute__((aligned(16))) float slots[TWPB][32 * TPITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, ql = lane & 31;
  const int64_t b = blockIdx.z, h = blockIdx.y;
  const int64_t q0 = ((int64_t)blockIdx.x * TWPB + wave) * 32;
  if (q0 >= p.T) return;                      // whole wave; no workgroup barrier below
  const int gh = p.grid_h, gw = p.grid_w, D = (int)p.D;
  const int nq = (int)(p.T - q0 < 32 ? p.T - q0 : 32);
  float* slot = slots[wave];
  // Q^T operand: column ql = token q0 + ql (zero past the end), dims 16c + 8g ..
  e8 qf[NC];
  {
    const E* qp = (const E*)p.q + b * p.q_sb + h * p.q_sh + (q0 + (ql < nq ? ql : 0)) * p.q_st + 8 * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = ql < nq ? *(const e8*)(qp + 16 * c) : (e8){};
  }
  const int64_t qlast = q0 + nq - 1;
  const int row0 = (int)(q0 / gw), row1 = (int)(qlast / gw);
  const int col0 = (int)(q0 % gw), col1 = (int)(qlast % gw);
  // Table operands of up to four 32-row blocks, loaded together (one memory
  // round trip; the rel_pos_w set goes out while the term_h rows are written).
  e8 tf[TRMAX / 32][NC];
  auto load_table = [&](const E* tab, int ntab, int r0, int nr) {
#pragma unroll
    for (int rb = 0; rb < TRMAX / 32; ++rb) {
      const int rl = rb * 32 + ql, r = r0 + rl;
      const bool ok = rl < nr && r < ntab;
      const E* tp = tab + (int64_t)(ok ? r : 0) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < NC; ++c) tf[rb][c] = (rb * 32 < nr && ok) ? *(const e8*)(tp + 16 * c) : (e8){};
    }
  };
  // Products over table rows r0 .. r0 + nr - 1 into the slot: slot[i][r - r0] = q_i . table[r].
  auto products = [&](int nr) {
#pragma unroll
    for (int rb = 0; rb < TRMAX / 32; ++rb) {
      if (rb * 32 >= nr) break;
      f32x16_t acc = (f32x16_t){};
#pragma unroll
      for (int c = 0; c < NC; ++c) acc = mfma32(tf[rb][c], qf[c], acc);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(f32x4_t*)(slot + ql * TPITCH + rb * 32 + 8 * i4 + 4 * g) =
            (f32x4_t){acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]};
    }
  };
  // Term rows of the block's tokens: out[i, y] = slot[i][base(i) - y],
  // base(i) = coord(i) + G - 1 - r0; nq x nout contiguous floats.  Lane l
  // writes elements e = W l, W l + 64 W, ... (W = 4 with 16-byte stores, else
  // 1); its token index q = e / nout, offset y and grid coordinates advance by
  // fixed steps, so only the first position takes a division.
  const float rcp_gw = 1.0f / (float)gw;
  auto read_out = [&](float* out, int nout, int G, int r0, bool by_row) {
    const int total = nq * nout;
    if ((256 % nout) == 0 && (nout & 3) == 0) {
      // nout divides the 256 floats one 16-byte store per lane covers: the
      // lane's offset y stays fixed and its token advances by 256 / nout per
      // step.  Four steps' slot reads go out before their stores.
      const int dqs = 256 / nout, y = (4 * lane) % nout, qb = (4 * lane) / nout;
      const int steps = (32 * nout + 255) / 256;         // 32 tokens x nout floats, 256 per step
#pragma unroll
      for (int k0 = 0; k0 < 32; k0 += 4) {
        if (k0 >= steps) break;
        f32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = qb + (k0 + u) * dqs;
          const int tq = (int)(q0 % gw) + q;             // token offset from the start of q0's grid row
          // tq / gw, exact: tq < 2^20 and gw <= 1024 keep the float quotient
          // far from the next integer (the 0.5 margin)
          const int drow = (int)(((float)tq + 0.5f) * rcp_gw);
          const int coord = by_row ? row0 + drow : tq - drow * gw;
          const float* sp = slot + (q < nq ? q : 0) * TPITCH + coord + G - 1 - r0 - y;
          v[u] = (f32x4_t){sp[0], sp[-1], sp[-2], sp[-3]};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = qb + (k0 + u) * dqs;
          if (k0 + u < steps && q < nq) *(f32x4_t*)(out + q * nout + y) = v[u];
        }
      }
      return;
    }
    const int W = (nout & 3) == 0 ? 4 : 1;
    const int stride = 64 * W;
    int e = W * lane;
    int q = e / nout, y = e - q * nout;
    const int dq = stride / nout, dy = stride - dq * nout;
    int row = (int)((q0 + q) / gw), col = (int)((q0 + q) % gw);
    for (; e < total; e += stride) {
      const float* sp = slot + q * TPITCH + (by_row ? row : col) + G - 1 - r0 - y;
      if (W == 4) *(f32x4_t*)(out + e) = (f32x4_t){sp[0], sp[-1], sp[-2], sp[-3]};
      else out[e] = sp[0];
      int adv = dq;
      y += dy;
      if (y >= nout) {
        y -= nout;
        ++adv;
      }
      q += adv;
      col += adv;
      while (col >= gw) {
        col -= gw;
        ++row;
      }
    }
  };
  const int64_t row_first = (b * p.H + h) * p.T + q0;
  const bool one_row = row0 == row1;
  const int r0h = row0, nrh = row1 - row0 + gh;
  const int r0w = one_row ? col0 : 0, nrw = one_row ? col1 - col0 + gw : 2 * gw - 1;
  load_table((const E*)p.rel_h, 2 * gh - 1, r0h, nrh);
  products(nrh);
  load_table((const E*)p.rel_w, 2 * gw - 1, r0w, nrw);
  wave_sync();
  read_out(p.term_h + row_first * gh, gh, gh, r0h, true);
  wave_sync();                                // slot reads done before the next products
  products(nrw);
  wave_sync();
  read_out(p.term_w + row_first * gw, gw, gw, r0w, false);
}

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

// The matrix-core kernel's conditions: 16-bit inputs, head_dim a multiple of
// 32 up to 128, 16-byte aligned rows, and products that fit the slot.
static bool terms_mfma_ok(const TermsParams& p) {
  if (!p.use_mfma || (p.dtype != 1 && p.dtype != 2) || (p.D != 32 && p.D != 64 && p.D != 128)) return false;
  if (terms_rows_h(p.grid_h, p.grid_w) > TRMAX || terms_rows_w(p.grid_w) > TRMAX) return false;
  if ((p.q_st % 8) != 0 || (((uintptr_t)p.q | (uintptr_t)p.rel_h | (uintptr_t)p.rel_w) & 15) != 0) return false;
  if (((uintptr_t)p.term_h | (uintptr_t)p.term_w) & 15) return false;
  return (p.T + 32 * TWPB - 1) / (32 * TWPB) <= 0x7fffffff && p.H <= 65535 && p.B <= 65535;
}

template <typename E>
static void launch_terms_mfma(const TermsParams& p, hipStream_t s) {
  dim3 grid((unsigned)((p.T + 32 * TWPB - 1) / (32 * TWPB)), (unsigned)p.H, (unsigned)p.B);
  if (p.D == 32) hipLaunchKernelGGL((relpos_terms_mfma_kernel<E, 2>), grid, dim3(64 * TWPB), 0, s, p);
  else if (p.D == 64) hipLaunchKernelGGL((relpos_terms_mfma_kernel<E, 4>), grid, dim3(64 * TWPB), 0, s, p);
  else hipLaunchKernelGGL((relpos_terms_mfma_kernel<E, 8>), grid, dim3(64 * TWPB), 0, s, p);
}

hipError_t launch_relpos_terms(const TermsParams& p, hipStream_t s) {
  if (terms_mfma_ok(p)) {
    if (p.dtype == 2) launch_terms_mfma<_Float16>(p, s);
    else launch_terms_mfma<__bf16>(p, s);
    return hipGetLastError();
  }
  dim3 grid((unsigned)p.grid_h, (unsigned)p.H, (unsigned)p.B);
  if (p.dtype == 0) launch_terms_typed<float>(p, grid, s);
  else if (p.dtype == 2) launch_terms_typed<_Float16>(p, grid, s);
  else launch_terms_typed<__bf16>(p, grid, s);
  return hipGetLastError();
}

}  // namespace sdpa
