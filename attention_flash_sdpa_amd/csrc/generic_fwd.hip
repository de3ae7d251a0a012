// Generic fused attention on the vector ALUs: any head_dim up to 128, fp32,
// bf16 or fp16 inputs, every bias kind, optional attention dropout.  It serves the fp32 path and shapes that the
// MFMA kernels do not cover.
//
// One query row per lane, 64 query rows per workgroup.  Small launches (fewer
// workgroups than compute units) give each workgroup four waves that split
// the key range between them: each wave runs the online softmax over its own
// key tiles and the four partial results (running max m, sum l, unnormalised
// output) are merged through LDS at the end.  K/V tiles are staged through
// LDS as fp32, per wave (rel-pos: each lane's term rows too, shared by the
// waves, formed here from the tables when the grid is small); each lane
// keeps its query row and output accumulator in registers and runs the online
// softmax (the accumulator is rescaled by exp(m_old - m_new) when the max
// grows), so no score row is ever stored.
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

// Key tile of one wave, and the words one wave needs: its K and V tiles and
// its score block while it runs, then its (m, l, output) rows for the merge.
template <int DMAX, int NW> struct GenericShape {
  static constexpr int BK = NW == 1 ? 32 : 16;
  static constexpr int TILE_F = 2 * BK * DMAX + BK * 64;
  static constexpr int MERGE_F = NW == 1 ? 0 : DMAX * 64 + 2 * 64;
  static constexpr int WF = TILE_F > MERGE_F ? TILE_F : MERGE_F;
};

template <typename TIN, int DMAX, int GF, int NW>
__global__ __launch_bounds__(64 * NW) void generic_fwd_kernel(FwdParams p) {
  typedef GenericShape<DMAX, NW> S;
  constexpr int BK = S::BK;
  __shared__ __attribute__((aligned(16))) float wsm[NW][S::WF];
  // Rel-pos: each lane's term_h row (grid_h values) and term_w row (grid_w
  // values) in LDS, [grid_h + grid_w][64 lanes]; with the fused terms the two
  // tables follow ([2 grid_h - 1 + 2 grid_w - 1][D]).
  extern __shared__ float dyn[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float(*ks)[DMAX] = (float(*)[DMAX])wsm[w];
  float(*vs)[DMAX] = (float(*)[DMAX])(wsm[w] + BK * DMAX);
  float(*zs)[64] = (float(*)[64])(wsm[w] + 2 * BK * DMAX);
  const int64_t b = blockIdx.z, h = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t i = i0 + lane;
  const bool live = i < p.Tq;
  const int D = (int)p.D;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const TIN* qp = (const TIN*)p.q + b * p.q_sb + h * p.q_sh + (live ? i : 0) * p.q_st;
  const TIN* kp = (const TIN*)p.k + b * p.k_sb + hk * p.k_sh;
  const TIN* vp = (const TIN*)p.v + b * p.k_sb + hk * p.k_sh;

  // (qp points at a valid row for every lane, so the loads need no lane test)
  float qr[DMAX], acc[DMAX];
#pragma unroll
  for (int c = 0; c < DMAX; ++c) {
    qr[c] = (D == DMAX || c < D) ? to_f32(qp[c]) : 0.0f;
    acc[c] = 0.0f;
  }
#pragma unroll
  for (int c = 0; c < DMAX; ++c) qr[c] = live ? qr[c] : 0.0f;
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
  const int gh = p.grid_h, gw = p.grid_w;
  // Dropout keep bits of this lane's score row (nullptr: no dropout).
  const uint32_t* krow = p.keep ? p.keep + ((b * p.Hq + h) * p.Tq + (live ? i : 0)) * p.keep_words : nullptr;
  // Grids too large for LDS rows read the workspace terms from memory.
  const bool rows_in_lds = (GF == GF_RELPOS) && (p.relpos_rows_lds != 0);
  const float* thg = nullptr;
  const float* twg = nullptr;
  if (GF == GF_RELPOS && !rows_in_lds) {
    const int64_t is = live ? i : 0;
    thg = p.term_h + ((b * p.Hq + h) * p.Tq + is) * gh;
    twg = p.term_w + ((b * p.Hq + h) * p.Tq + is) * gw;
  }
  // Copies into LDS that issue 8 loads per lane before the first store (one
  // memory round trip per batch): rows w, w + NW, ... of a lane's own row of
  // n values to dst[e * 64], and a cooperative copy of n elements to dst[e].
  constexpr int NB = 8;
  auto copy_row = [&](float* dst, const float* src, int n) {
    for (int e0 = w; e0 < n; e0 += NB * NW) {
      float v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) v[u] = e0 + u * NW < n ? src[e0 + u * NW] : 0.0f;
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (e0 + u * NW < n) dst[(e0 + u * NW) * 64] = v[u];
    }
  };
  // Both tables in one pass: dst[0, n0) from src0, dst[n0, n0 + n1) from src1.
  auto copy_all = [&](float* dst, const TIN* src0, int n0, const TIN* src1, int n1) {
    const int n = n0 + n1;
    for (int e0 = 0; e0 < n; e0 += NB * 64 * NW) {
      float v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = e0 + 64 * NW * u + (int)threadIdx.x;
        v[u] = e < n0 ? to_f32(src0[e]) : (e < n ? to_f32(src1[e - n0]) : 0.0f);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = e0 + 64 * NW * u + (int)threadIdx.x;
        if (e < n) dst[e] = v[u];
      }
    }
  };
  // Tile copies.  With D == DMAX and 16-byte aligned rows every lane moves
  // whole 16-byte pieces, all loads of a tile issued before any LDS store (one
  // memory round trip per tile), and with few pieces per lane the next tile's
  // loads go out before this tile's arithmetic (the first tile's before the
  // rel-pos staging); other shapes copy element by element.  Wave w takes key
  // tiles w, w + NW, ...; its buffers are its own, so a wave-level order is
  // all the copies need.
  constexpr int EPP = 16 / sizeof(TIN);               // elements per 16-byte piece
  constexpr int NPC = BK * DMAX / EPP;                // pieces per tensor per tile
  constexpr int PPL = (NPC + 63) / 64;                // pieces per lane per tensor
  constexpr bool AHEAD = PPL <= 4;                    // registers for a tile in flight
  typedef TIN tin16 __attribute__((ext_vector_type(EPP)));
  const bool vec = D == DMAX && (p.k_st % EPP) == 0 && (((uintptr_t)kp | (uintptr_t)vp) & 15) == 0;
  const int64_t jstep = (int64_t)NW * BK;
  tin16 kr[PPL], vr[PPL];
  auto load_tile = [&](int64_t j0) {
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int e = lane + 64 * u, jj = e / (DMAX / EPP), c = (e % (DMAX / EPP)) * EPP;
      const int64_t j = j0 + jj;
      const bool ok = (NPC % 64 == 0 || e < NPC) && j < hi;
      kr[u] = ok ? *(const tin16*)(kp + j * p.k_st + c) : (tin16){};
      vr[u] = ok ? *(const tin16*)(vp + j * p.k_st + c) : (tin16){};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int e = lane + 64 * u, jj = e / (DMAX / EPP), c = (e % (DMAX / EPP)) * EPP;
      if (NPC % 64 == 0 || e < NPC) {
#pragma unroll
        for (int x = 0; x < EPP; ++x) {
          ks[jj][c + x] = to_f32(kr[u][x]);
          vs[jj][c + x] = to_f32(vr[u][x]);
        }
      }
    }
  };
  const int64_t jfirst = lo + (int64_t)w * BK;
  if (AHEAD && vec && jfirst < hi) load_tile(jfirst);

  if (rows_in_lds) {
    const int64_t is = live ? i : 0;
    if (p.term_h) {                   // terms from the workspace: this lane's rows, one value per LDS row
      const float* th = p.term_h + ((b * p.Hq + h) * p.Tq + is) * gh;
      const float* tw = p.term_w + ((b * p.Hq + h) * p.Tq + is) * gw;
      copy_row(dyn + lane, th, gh);
      copy_row(dyn + gh * 64 + lane, tw, gw);
    } else {                          // terms formed here: term[i, y] = q_i . table[coord(i) - y + G - 1]
      float* tab = dyn + (gh + gw) * 64;
      const int nh = 2 * gh - 1, nw = 2 * gw - 1;
      // [nh + nw][D]: rel_pos_h rows then rel_pos_w rows, both stored row-major
      copy_all(tab, (const TIN*)p.rel_h, nh * D, (const TIN*)p.rel_w, nw * D);
      __syncthreads();
      const int ih = (int)(is / gw), iw = (int)(is % gw);
      auto dotrow = [&](const float* row) -> float {
        float d = 0.0f;
        if (D == DMAX) {
#pragma unroll
          for (int c = 0; c < DMAX; ++c) d = fmaf(qr[c], row[c], d);
        } else {
#pragma unroll
          for (int c = 0; c < DMAX; ++c) d = (c < D) ? fmaf(qr[c], row[c], d) : d;
        }
        return d;
      };
      for (int y = w; y < gh; y += NW) dyn[y * 64 + lane] = dotrow(tab + (ih - y + gh - 1) * D);
      for (int x = w; x < gw; x += NW) dyn[(gh + x) * 64 + lane] = dotrow(tab + (nh + iw - x + gw - 1) * D);
    }
    __syncthreads();                  // every wave reads every row
  }

  for (int64_t j0 = jfirst; j0 < hi; j0 += jstep) {
    wave_sync();                      // this wave's reads of the previous tile are done
    if (vec) {
      if (!AHEAD) load_tile(j0);
      store_tile();
      if (AHEAD && j0 + jstep < hi) load_tile(j0 + jstep);
    } else {
      for (int e = lane; e < BK * DMAX; e += 64) {
        const int jj = e / DMAX, c = e % DMAX;
        const int64_t j = j0 + jj;
        const bool ok = j < hi && c < D;
        ks[jj][c] = ok ? to_f32(kp[j * p.k_st + c]) : 0.0f;
        vs[jj][c] = ok ? to_f32(vp[j * p.k_st + c]) : 0.0f;
      }
    }
    wave_sync();                      // the tile is in LDS for every lane of the wave
    const int nk = (int)((hi - j0 < BK) ? hi - j0 : BK);
    float tmax = -INFINITY;
    int jh = 0, jw = 0;                 // grid row and column of key j0 + jj
    if (GF == GF_RELPOS) {
      jh = (int)(j0 / gw);
      jw = (int)(j0 % gw);
    }
#pragma unroll 2
    for (int jj = 0; jj < nk; ++jj) {
      const int64_t j = j0 + jj;
      float d = 0.0f;
#pragma unroll
      for (int c = 0; c < DMAX; ++c) d = fmaf(qr[c], ks[jj][c], d);
      float z = d * p.scale;
      bool ok = live;
      if (GF == GF_INDEX) ok = ok && index_allowed(p.bias, i, j, p.offset, p.window);
      if (GF == GF_RELPOS) {
        z += rows_in_lds ? dyn[jh * 64 + lane] + dyn[(gh + jw) * 64 + lane] : thg[jh] + twg[jw];
        if (++jw == gw) {
          jw = 0;
          ++jh;
        }
      }
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
        // dropout: the row sum takes every weight, P.V only the kept ones
        // (the common factor of kept weights is applied at the end)
        float pv = pj;
        if (krow) {
          const int64_t j = j0 + jj;
          pv = ((krow[j >> 5] >> (j & 31)) & 1u) ? pj : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < DMAX; ++c) acc[c] = fmaf(pv, vs[jj][c], acc[c]);
      }
    }
  }
  // Channels this wave writes: all of them with one wave; with several, the
  // partial results meet in LDS and wave w merges and writes channels
  // [w DMAX / NW, (w + 1) DMAX / NW) of every row.
  constexpr int CPW = DMAX / NW;
  float out[CPW];
  if (NW == 1) {
#pragma unroll
    for (int c = 0; c < CPW; ++c) out[c] = acc[c];
  } else {
    __syncthreads();                  // every wave is done with its tiles
    float* mine = wsm[w];
    mine[lane] = m;
    mine[64 + lane] = l;
#pragma unroll
    for (int c = 0; c < DMAX; ++c) mine[128 + c * 64 + lane] = acc[c];
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, wsm[v][lane]);
    float L = 0.0f;
#pragma unroll
    for (int c = 0; c < CPW; ++c) out[c] = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {      // fixed order: the result does not depend on timing
      const float mv = wsm[v][lane];
      const float f = (mv == -INFINITY) ? 0.0f : expf(mv - M);
      L = fmaf(f, wsm[v][64 + lane], L);
#pragma unroll
      for (int c = 0; c < CPW; ++c) out[c] = fmaf(f, wsm[v][128 + (w * CPW + c) * 64 + lane], out[c]);
    }
    m = M;
    l = L;
  }
  if (!live) return;
  const float inv = (l > 0.0f) ? (krow ? p.keep_scale : 1.0f) / l : 0.0f;
  const int64_t ob = b * p.q_sb + h * p.q_sh + i * p.q_st + w * CPW;
  const int cn = D - w * CPW;           // channels of this wave's slice that exist
  if (p.out_dtype == 0) {
    float* op = (float*)p.o + ob;
#pragma unroll
    for (int c = 0; c < CPW; ++c) if (c < cn) op[c] = out[c] * inv;
  } else {                            // 16-bit output in the input's type
    TIN* op = (TIN*)p.o + ob;
#pragma unroll
    for (int c = 0; c < CPW; ++c) if (c < cn) op[c] = (TIN)(out[c] * inv);
  }
  if (p.lse && w == 0) p.lse[(b * p.Hq + h) * p.Tq + i] = (l > 0.0f) ? m + logf(l) : -INFINITY;
}

// Bytes of dynamic LDS for rel-pos: per-lane term rows, plus the tables when
// the terms are formed in the kernel.
static size_t relpos_lds(const FwdParams& p, bool fused) {
  size_t n = (size_t)(p.grid_h + p.grid_w) * 64;
  if (fused) n += (size_t)(2 * p.grid_h - 1 + 2 * p.grid_w - 1) * p.D;
  return n * sizeof(float);
}

static int dmax_of(int64_t D) { return D <= 16 ? 16 : D <= 32 ? 32 : D <= 64 ? 64 : 128; }

// Static LDS of one instance: each wave's K and V tiles and score block (or
// its merge rows).
static size_t static_lds(int64_t D, int nw) {
  const int dm = dmax_of(D);
  const int bk = nw == 1 ? 32 : 16;
  const size_t tile = (size_t)2 * bk * dm + (size_t)bk * 64, merge = nw == 1 ? 0 : (size_t)dm * 64 + 128;
  return (size_t)nw * (tile > merge ? tile : merge) * 4;
}

// Four waves per workgroup when the launch has fewer workgroups than the GPU
// has compute units, head_dim is at most 32 and the key range spans more than
// one 16-key tile (unless switched off); one wave otherwise.
static int waves_of(const FwdParams& p, size_t dyn_lds) {
  const int64_t blocks = (p.Tq + 63) / 64 * p.Hq * p.B;
  if (!p.generic_multiwave || p.D > 32 || blocks >= 256 || p.Tkv <= 16) return 1;
  return static_lds(p.D, 4) + dyn_lds <= 64 * 1024 ? 4 : 1;
}

template <typename TIN, int DMAX, int GF>
static void launch_gf(const FwdParams& p, dim3 grid, size_t dyn, hipStream_t s) {
  if (DMAX <= 32 && waves_of(p, dyn) == 4)
    hipLaunchKernelGGL((generic_fwd_kernel<TIN, DMAX, GF, (DMAX <= 32 ? 4 : 1)>), grid, dim3(256), dyn, s, p);
  else
    hipLaunchKernelGGL((generic_fwd_kernel<TIN, DMAX, GF, 1>), grid, dim3(64), dyn, s, p);
}

template <typename TIN, int DMAX>
static void launch_dim(const FwdParams& p, dim3 grid, hipStream_t s) {
  switch (p.bias) {
    case BIAS_NONE: launch_gf<TIN, DMAX, GF_NONE>(p, grid, 0, s); break;
    case BIAS_CAUSAL:
    case BIAS_SLIDING: launch_gf<TIN, DMAX, GF_INDEX>(p, grid, 0, s); break;
    case BIAS_RELPOS: {
      FwdParams q = p;
      q.relpos_rows_lds = generic_relpos_supported(p, !p.term_h) ? 1 : 0;
      launch_gf<TIN, DMAX, GF_RELPOS>(q, grid, q.relpos_rows_lds ? relpos_lds(p, !p.term_h) : 0, s);
      break;
    }
    default: launch_gf<TIN, DMAX, GF_TENSOR>(p, grid, 0, s); break;
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

bool generic_relpos_supported(const FwdParams& p, bool fused) {
  return p.grid_h >= 1 && p.grid_w >= 1 && static_lds(p.D, 1) + relpos_lds(p, fused) <= 64 * 1024;
}

hipError_t launch_generic_fwd(const FwdParams& p, hipStream_t s) {
  if (p.dtype == 0) return launch_typed<float>(p, s);
  return p.dtype == 2 ? launch_typed<_Float16>(p, s) : launch_typed<__bf16>(p, s);
}

}  // namespace sdpa
