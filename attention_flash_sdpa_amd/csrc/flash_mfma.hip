// Flash attention forward on gfx950 bf16 matrix cores (MFMA 32x32x16).
//
//   O = softmax(Q . K^T * scale + B) . V      ([Axon PR 650]
//   "Axon.Layers.scaled_dot_product_attention/4", description)
//
// computed tile by tile with an online softmax, so no T_q x T_kv array is
// written.  Optional attention dropout (keep bits per score, [Axon PR 650],
// description: dropout in :train mode): the row sum takes every weight and
// P.V only the kept ones, and the output is multiplied by the kept-weight
// factor at the end.  Bias kinds: none, causal / sliding-window (index masks, with
// tile skipping), additive / boolean tensors (through broadcast strides), and
// SAM's decomposed rel-pos bias rebuilt in registers from the per-query
// term rows ([Candle PR 3280] "feat(metal): SDPA with Relative Positional
// Embeddings & LayerNorm Stability", Key Changes; [mlx-examples issue 1451]
// "segment_anything: fuse attention with mx.fast.scaled_dot_product_attention",
// body).
//
// Work split.  A workgroup is 4 waves; each wave owns 32 query rows of one
// head.  With grouped-query attention the waves of a workgroup are the query
// heads that share one KV head (same 32 positions), so one K/V tile in LDS
// feeds all of them and their mask patterns coincide.  Without sharing the
// waves take 4 consecutive 32-row blocks of one head.
//
// Per 64-key tile and wave:
//   S^T[key, q] = K . Q^T        2 key blocks x D/16 MFMAs; K from LDS
//                                (ds_read_b128), Q^T held in registers.
//                                The transposed orientation puts one query
//                                per lane, so the row max and sum of the
//                                softmax are in-lane plus one lane swap.
//   x = S^T * scale * log2(e) + bias * log2(e)   (log2 domain, exp2 below)
//   online softmax: the running max is only moved when a tile's max exceeds
//                   it by more than 8 (log2 units); otherwise probabilities up
//                   to 2^8 are accumulated against the old max, which is
//                   exact after the final division and skips most rescales.
//   O^T[d, q] += V^T . P^T       D/32 row blocks x 4 MFMAs; P^T comes straight
//                                from the S^T registers (bf16), V^T from LDS
//                                through the gfx950 transposing LDS read
//                                (ds_read_b64_tr_b16) on the row-major V tile.
//
// Rel-pos with a 64-wide grid row (the key tile = one grid row): the
// term_w[q, col] / scale values for the 64 key columns are the same for every
// tile, so they initialise the S^T accumulators of the first MFMA of each key
// block (zero VALU cost), and term_h[q, row] is one scalar per query per tile
// folded into the exponent's offset.
//
// Fused rel-pos (64-wide grid rows, head_dim 64): the workgroup forms the
// terms itself from its Q tile and the tables, so no term array exists:
//   term_h for the wave's 32 queries (one grid row r) is one small GEMM
//     TH^T[y, q] = sum_c rel_pos_h[r + grid_h - 1 - y, c] * Q[q, c]
//   on the matrix cores, kept in LDS as [y][q] and read once per tile;
//   term_w[q, x] = q . rel_pos_w[col(q) - x + 63] is the skewed diagonal of
//     AW^T[m, q] = sum_c rel_pos_w[m, c] * Q[q, c]  (m = col - x + 63),
//   formed by MFMA over the 96 table rows the wave can touch, then gathered
//   along the skew through LDS into the accumulator-initialisation registers.
#include "common.h"

namespace sdpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // lazy-rescale threshold (log2 units)

enum Mode { M_NONE = 0, M_INDEX = 1, M_TENSOR = 2, M_RELPOS_ROW = 3, M_RELPOS_FUSED = 4 };

template <int D>
struct Cfg {
  static constexpr int BN = 64;                   // keys per tile
  static constexpr int PITCH = D * 2;             // LDS row pitch in bytes (rows unpadded; chunks XOR-swizzled)
  static constexpr int TILE = BN * PITCH;         // bytes of one K or V tile
  static constexpr int CH = D / 8;                // 16-byte chunks per row
  static constexpr int LOADS = BN * CH / 256;     // 16-byte global loads per thread per tile (K or V)
  static constexpr int QC = D / 16;               // MFMA k-chunks of Q.K^T
  static constexpr int DB = D / 32;               // 32-row blocks of O^T
  static constexpr int RPB = 256 / (2 * D);       // rows per 256-byte bank sweep (64 banks x 4 B)
  // 16-byte chunk c of K row r lives at chunk position c ^ kswz(r): the 16 rows
  // read by 16 lanes at one chunk index land in 16 distinct bank groups.
  static __device__ __forceinline__ int kswz(int r) { return (r / RPB) & (CH - 1); }
  // V rows are read 4 at a time, 64 contiguous bytes each (transposing reads):
  // flipping whole 64-byte groups per row keeps the 4 rows in distinct banks.
  static __device__ __forceinline__ int vswz(int r) { return ((r / RPB) % (4 / RPB)) << 2; }
};

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_char* p) {
  return *(const __attribute__((address_space(3))) bf16x8*)p;
}
__device__ __forceinline__ s16x4 lds_read_tr(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}
__device__ __forceinline__ void lds_write_b128(lds_char* p, bf16x8 v) {
  *(__attribute__((address_space(3))) bf16x8*)p = v;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Max / sum of the value held by lane l and lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float halves_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float halves_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Fused rel-pos prologue (head_dim 64, grid_w 64).  Forms term_w / scale for
// the wave's 32 queries in the accumulator layout (cinit) and writes term_h^T
// [y][q] into the wave's LDS slot after the K/V buffers.  Uses the K/V buffer
// space as scratch, so it runs before the first tile is staged.
template <int D>
__device__ __forceinline__ void relpos_prologue(const FwdParams& p, lds_char* smem, const bf16x8* qf, int wave,
                                                int lane, int64_t qw0, f32x16* cinit) {
  using C = Cfg<D>;
  const int g = lane >> 5, ql = lane & 31;
  const int gh = p.grid_h;
  const int64_t r = qw0 / 64;            // grid row of all 32 queries of this wave
  const int c0 = (int)(qw0 % 64);        // column of the wave's first query (0 or 32)
  const __bf16* rh = (const __bf16*)p.rel_h;
  const __bf16* rw = (const __bf16*)p.rel_w;
  // TH^T[y, q] for y = yb*32 + row: A rows are rel_pos_h[r + gh - 1 - y].
  f32x16 th[2];
#pragma unroll
  for (int yb = 0; yb < 2; ++yb) {
    th[yb] = (f32x16){};
    const int y = yb * 32 + ql;
    const int64_t tr = r + gh - 1 - y;
#pragma unroll
    for (int c = 0; c < C::QC; ++c) {
      bf16x8 a = (bf16x8){};
      if (y < gh) a = *(const bf16x8*)(rh + tr * D + c * 16 + 8 * g);
      th[yb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], th[yb], 0, 0, 0);
    }
  }
  // AW^T[m', q] = rel_pos_w[c0 + m'] . q for m' in [0, 96).
  f32x16 aw[3];
#pragma unroll
  for (int mb = 0; mb < 3; ++mb) {
    aw[mb] = (f32x16){};
    const int m = c0 + mb * 32 + ql;
#pragma unroll
    for (int c = 0; c < C::QC; ++c) {
      bf16x8 a = (bf16x8){};
      if (m < 127) a = *(const bf16x8*)(rw + (int64_t)m * D + c * 16 + 8 * g);
      aw[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], aw[mb], 0, 0, 0);
    }
  }
  // Skewed gather through LDS: slot per wave [32 q][97] fp32 (odd pitch: conflict-free).
  typedef __attribute__((address_space(3))) float lds_float;
  lds_float* slot = (lds_float*)(smem + wave * (32 * 97 * 4));
#pragma unroll
  for (int mb = 0; mb < 3; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) slot[ql * 97 + mb * 32 + 8 * (i / 4) + 4 * g + (i % 4)] = aw[mb][i];
  __syncthreads();
  const float inv_scale = 1.0f / p.scale;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int x = kb * 32 + 8 * (i / 4) + 4 * g + (i % 4);
      cinit[kb][i] = slot[ql * 97 + ql + 63 - x] * inv_scale;     // m' = col - x + 63 - c0 = ql + 63 - x
    }
  __syncthreads();
  lds_float* ths = (lds_float*)(smem + 4 * C::TILE + wave * (64 * 32 * 4));
#pragma unroll
  for (int yb = 0; yb < 2; ++yb)
#pragma unroll
    for (int i = 0; i < 16; ++i) ths[(yb * 32 + 8 * (i / 4) + 4 * g + (i % 4)) * 32 + ql] = th[yb][i];
}

template <int D, int MODE, bool OUT_BF16, bool DROP>
__global__ __launch_bounds__(256, 2) void flash_mfma_kernel(FwdParams p, int hpw) {
  using C = Cfg<D>;
  // Software pipelining (next tile's scores in flight during this tile's
  // softmax) needs a second score tile in registers: affordable at head_dim 64.
  constexpr bool PIPE = false;
  // K/V double buffer, then (fused rel-pos) per-wave term_h^T [64 y][32 q] fp32.
  constexpr int TH_BYTES = (MODE == M_RELPOS_FUSED) ? 4 * 64 * 32 * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem_raw[4 * C::TILE + TH_BYTES];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform (scalar) index
  const int g = lane >> 5;            // lane half: selects rows of the MFMA layouts
  const int ql = lane & 31;           // query column of this lane
  const int nqb = 4 / hpw;            // 32-row query blocks per workgroup
  // Workgroups are dealt to the 8 XCDs round-robin by linear id; renumber them
  // so that each XCD gets a contiguous range of (batch, head, query tile) and
  // keeps its heads' K/V resident in its own L2.
  const int64_t nblk = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int64_t lin = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t per = nblk / 8, rem = nblk % 8, xcd = lin % 8;
  const int64_t lid = xcd * per + min(xcd, rem) + lin / 8;
  const int64_t bx = lid % gridDim.x, by = (lid / gridDim.x) % gridDim.y, bz = lid / ((int64_t)gridDim.x * gridDim.y);
  const int64_t b = bz;
  const int64_t qtile = (MODE == M_INDEX) ? (int64_t)(gridDim.x - 1 - bx) : bx;
  const int64_t h = by * hpw + (wave % hpw);
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t wg_q0 = qtile * 32 * nqb;
  const int64_t wg_q1 = min(wg_q0 + 32 * nqb, p.Tq) - 1;
  const int64_t wq0 = wg_q0 + 32 * (wave / hpw);
  const int64_t wq1 = min(wq0 + 31, p.Tq - 1);
  const int64_t qrow = wq0 + ql;
  const bool qvalid = qrow < p.Tq;
  const int64_t qsafe = qvalid ? qrow : 0;

  const __bf16* qp = (const __bf16*)p.q + b * p.q_sb + h * p.q_sh;
  const __bf16* kp = (const __bf16*)p.k + b * p.k_sb + hk * p.k_sh;
  const __bf16* vp = (const __bf16*)p.v + b * p.k_sb + hk * p.k_sh;

  // Q^T as the B operand: lane holds query ql, head dims c*16 + 8*g .. +7.
  bf16x8 qf[C::QC];
#pragma unroll
  for (int c = 0; c < C::QC; ++c) {
    if (qvalid) qf[c] = *(const bf16x8*)(qp + qrow * p.q_st + c * 16 + 8 * g);
    else qf[c] = (bf16x8){};
  }

  // Key range of the workgroup.
  int64_t lo = 0, hi = p.Tkv;
  if (MODE == M_INDEX) {
    hi = min(hi, wg_q1 + p.offset + 1);
    if (p.bias == BIAS_SLIDING) lo = max((int64_t)0, wg_q0 + p.offset - p.window + 1);
  }
  const int64_t t0 = lo / C::BN;
  const int ntiles = hi > lo ? (int)((hi - t0 * C::BN + C::BN - 1) / C::BN) : 0;

  const float c2 = p.scale * kLog2e;

  // Rel-pos (64-wide grid rows): term_w / scale initialises the score accumulators.
  f32x16 cinit[2];
  const float* thp = nullptr;
  if (MODE == M_RELPOS_ROW) {
    const float inv_scale = 1.0f / p.scale;
    const float* twp = p.term_w + ((b * p.Hq + h) * p.Tq + qsafe) * 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 t = *(const f32x4*)(twp + kb * 32 + 8 * i4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) cinit[kb][4 * i4 + e] = t[e] * inv_scale;
      }
    thp = p.term_h + ((b * p.Hq + h) * p.Tq + qsafe) * p.grid_h;
  } else if (MODE == M_RELPOS_FUSED) {
    relpos_prologue<D>(p, smem, qf, wave, lane, wq0, cinit);
  } else {
    cinit[0] = (f32x16){};
    cinit[1] = (f32x16){};
  }
  const lds_char* th_lds = smem + 4 * C::TILE + wave * (64 * 32 * 4) + ql * 4;

  f32x16 o[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) o[d] = (f32x16){};
  float m = -INFINITY, l = 0.0f;

  // LDS rings: K tiles run one tile ahead of V tiles.  Iteration `it` reads
  // K_{it+1} (scores of the next tile, issued to the matrix cores before the
  // softmax of this tile so the two overlap) and V_it (P.V of this tile); it
  // stages K_{it+2} and V_{it+1} from HBM into the buffers freed by the
  // previous iteration.
  auto kbuf = [&](int i) -> lds_char* { return smem + (i & 1) * C::TILE; };
  auto vbuf = [&](int i) -> lds_char* { return smem + (2 + (i & 1)) * C::TILE; };
  bf16x8 kst[C::LOADS], vst[C::LOADS];
  auto gload = [&](const __bf16* src, int64_t k0, bf16x8* dst) {
    if (k0 + C::BN <= p.Tkv) {          // whole tile in range: no per-load predicate
#pragma unroll
      for (int r = 0; r < C::LOADS; ++r) {
        const int cidx = tid + 256 * r;
        const int row = cidx / C::CH, col = cidx % C::CH;
        dst[r] = *(const bf16x8*)(src + (k0 + row) * p.k_st + col * 8);
      }
    } else {
#pragma unroll
      for (int r = 0; r < C::LOADS; ++r) {
        const int cidx = tid + 256 * r;
        const int row = cidx / C::CH, col = cidx % C::CH;
        const int64_t key = k0 + row;
        dst[r] = (key < p.Tkv) ? *(const bf16x8*)(src + key * p.k_st + col * 8) : (bf16x8){};
      }
    }
  };
  auto lstore = [&](lds_char* dstbuf, const bf16x8* src, bool is_v) {
#pragma unroll
    for (int r = 0; r < C::LOADS; ++r) {
      const int cidx = tid + 256 * r;
      const int row = cidx / C::CH, col = cidx % C::CH;
      const int pos = col ^ (is_v ? C::vswz(row) : C::kswz(row));
      lds_write_b128(dstbuf + row * C::PITCH + pos * 16, src[r]);
    }
  };
  // Tile classes for this wave: skip (no allowed key) / partial (per-element test) / full.
  auto tile_skip = [&](int64_t k0) -> bool {
    if (MODE != M_INDEX) return false;
    const int64_t klast = k0 + C::BN - 1;
    if (k0 > wq1 + p.offset) return true;
    if (p.bias == BIAS_SLIDING && klast <= wq0 + p.offset - p.window) return true;
    return false;
  };
  auto tile_partial = [&](int64_t k0) -> bool {
    bool part = (k0 + C::BN > p.Tkv) || (MODE == M_TENSOR);
    if (MODE == M_INDEX) {
      if (k0 + C::BN - 1 > wq0 + p.offset) part = true;
      if (p.bias == BIAS_SLIDING && k0 <= wq1 + p.offset - p.window) part = true;
    }
    return part;
  };
  // S^T = K . Q^T (+ rel-pos accumulator initialisation) for the tile in `ks`.
  auto qk = [&](const lds_char* ks, f32x16* sc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = cinit[kb];
#pragma unroll
    for (int c = 0; c < C::QC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + ql;
        const bf16x8 a = lds_read_b128(ks + row * C::PITCH + ((2 * c + g) ^ C::kswz(row)) * 16);
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], sc[kb], 0, 0, 0);
      }
  };

  if (ntiles > 0) {
    gload(kp, t0 * C::BN, kst);
    gload(vp, t0 * C::BN, vst);
    lstore(kbuf(0), kst, false);
    lstore(vbuf(0), vst, true);
    if (PIPE && ntiles > 1) {
      gload(kp, (t0 + 1) * C::BN, kst);
      lstore(kbuf(1), kst, false);
    }
  }
  __syncthreads();

  // Allowed key interval of this lane's query: lim_lo < key <= lim_hi (int32).
  int lim_hi = (int)(p.Tkv - 1), lim_lo = -1;
  if (MODE == M_INDEX) {
    const int64_t hi64 = min(qrow + p.offset, p.Tkv - 1);
    lim_hi = (int)max(hi64, (int64_t)-2);
    if (p.bias == BIAS_SLIDING) lim_lo = (int)min(max(qrow + p.offset - p.window, (int64_t)-1), p.Tkv);
  }
  auto th_of = [&](int64_t tile) -> float {
    if (MODE == M_RELPOS_ROW) return thp[tile];
    if (MODE == M_RELPOS_FUSED) return *(const __attribute__((address_space(3))) float*)(th_lds + tile * 128);
    return 0.0f;
  };

  f32x16 s[2];
  s[0] = (f32x16){};
  s[1] = (f32x16){};
  if (PIPE && ntiles > 0 && !tile_skip(t0 * C::BN)) qk(kbuf(0), s);

  for (int it = 0; it < ntiles; ++it) {
    const int64_t k0 = (t0 + it) * C::BN;
    const bool stage_k = it + (PIPE ? 2 : 1) < ntiles, stage_v = it + 1 < ntiles;
    if (stage_k) gload(kp, k0 + (PIPE ? 2 : 1) * C::BN, kst);
    if (stage_v) gload(vp, k0 + C::BN, vst);
    const float th_cur = th_of(t0 + it);
    const bool skip = tile_skip(k0);
    const bool partial = tile_partial(k0);
    // Scores of the next tile go to the matrix cores first.
    f32x16 sn[2];
    sn[0] = (f32x16){};
    sn[1] = (f32x16){};
    if (PIPE) {
      if (it + 1 < ntiles && !tile_skip(k0 + C::BN)) qk(kbuf(it + 1), sn);
    } else if (!skip) {
      qk(kbuf(it), s);
    }

    if (!skip) {
      const lds_char* vs = vbuf(it);
      // Dropout keep bits of this lane's row for the tile's 64 keys (tiles start at multiples of 64).
      uint32_t kw[2] = {0u, 0u};
      if (DROP && qvalid) {
        const int64_t w0 = k0 / 32;
        const uint32_t* kr = p.keep + ((b * p.Hq + h) * p.Tq + qrow) * p.keep_words + w0;
        kw[0] = kr[0];
        kw[1] = (w0 + 1 < p.keep_words) ? kr[1] : 0u;
      }
      // Masks and tensor biases act on the raw scores (bias / scale), so every
      // mode shares one exponent: p = exp2(s * scale * log2e + (rowb - m)).
      if (MODE == M_TENSOR) {
        const float inv_scale = 1.0f / p.scale;
        const int msz = (p.bias == BIAS_BOOL) ? 1 : (p.mdtype == 0 ? 4 : 2);
        const int mstep = (int)p.ms[3] * msz;
        const char* mrow = (const char*)p.mdata +
                           (b * p.ms[0] + h * p.ms[1] + qsafe * p.ms[2] + (k0 + 4 * g) * p.ms[3]) * msz;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kofs = kb * 32 + 8 * (i / 4) + (i % 4);
            if (qvalid && k0 + 4 * g + kofs < p.Tkv) {
              const char* mp = mrow + kofs * mstep;
              float mv;
              if (msz == 1) mv = *(const uint8_t*)mp ? 0.0f : -INFINITY;
              else if (msz == 4) mv = *(const float*)mp;
              else mv = (float)*(const __bf16*)mp;
              s[kb][i] = fmaf(mv, inv_scale, s[kb][i]);
            }
          }
      }
      if (partial) {
        asm volatile("" ::: "memory");   // keep this a real branch: full tiles skip the mask work
        const int kl0 = (int)(k0 + 4 * g);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kl0 + kb * 32 + 8 * (i / 4) + (i % 4);
            const bool ok = (key <= lim_hi) & (key > lim_lo);
            s[kb][i] = ok ? s[kb][i] : -INFINITY;
          }
      }
      const float rowb = (MODE == M_RELPOS_ROW || MODE == M_RELPOS_FUSED) ? th_cur * kLog2e : 0.0f;
      float smax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) smax = max3f(smax, s[kb][i], s[kb][i + 1]);
      smax = halves_max(smax);
      const float tmax = fmaf(smax, c2, rowb);        // -inf stays -inf (c2 > 0)
      const bool need = tmax > m + kTau;
      if (__builtin_expect(__any(need), 0)) {
        const float mn = need ? tmax : m;
        const float alpha = need ? ((m == -INFINITY) ? 0.0f : fast_exp2(m - mn)) : 1.0f;
        m = mn;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < C::DB; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
      }
      const float off = rowb - ((m == -INFINITY) ? 0.0f : m);
      // P^T operands for the 4 PV MFMAs (16 keys each); the row sum adds the
      // bf16-rounded probabilities that the MFMA consumes (dot2 with ones).
      bf16x8 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x2 pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2 pp = {fast_exp2(fmaf(s[t / 2][8 * (t % 2) + e], c2, off)),
                            fast_exp2(fmaf(s[t / 2][8 * (t % 2) + e + 1], c2, off))};
          pk[e / 2] = __builtin_convertvector(pp, bf16x2);
          l = __builtin_amdgcn_fdot2_f32_bf16(pk[e / 2], kOnes2, l, false);
          if (DROP) {       // dropped weights leave P.V (the row sum above keeps them)
            const int i0 = 8 * (t % 2) + e;                      // even: i0 and i0 + 1 are adjacent keys
            const uint32_t two = (kw[t / 2] >> (8 * (i0 / 4) + 4 * g + (i0 % 4))) & 3u;
            const uint32_t msk = ((two & 1u) ? 0xFFFFu : 0u) | ((two & 2u) ? 0xFFFF0000u : 0u);
            pk[e / 2] = __builtin_bit_cast(bf16x2, __builtin_bit_cast(uint32_t, pk[e / 2]) & msk);
          }
        }
        pb[t] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                        __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      }
      // O^T += V^T . P^T with transposed LDS reads of the row-major V tile.
      const int j = lane & 15;
      const int dh = (lane >> 4) & 1;
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int col = d * 32 + 16 * dh + 4 * (j & 3);
          const int row0 = 16 * t + 4 * g + (j >> 2);
          // byte offset col*2 = 16 * chunk + 8 * ((j & 3) & 1); rows row0 and row0 + 8
          // have the same swizzle (the swizzle depends on row / RPB modulo 4 / RPB).
          const int chunk = (col * 2) >> 4, within = (col * 2) & 15;
          const int off = ((chunk ^ C::vswz(row0)) << 4) + within;
          const s16x4 lo4 = lds_read_tr(vs + row0 * C::PITCH + off);
          const s16x4 hi4 = lds_read_tr(vs + (row0 + 8) * C::PITCH + off);
          const s16x8 a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[t], o[d], 0, 0, 0);
        }
    }
    if (stage_k) lstore(kbuf(PIPE ? it : it + 1), kst, false);
    if (stage_v) lstore(vbuf(it + 1), vst, true);
    __syncthreads();
    if (PIPE) {
      s[0] = sn[0];
      s[1] = sn[1];
    }
  }

  // Epilogue: the two lane halves hold disjoint keys of the same query.
  const float lt = halves_sum(l);
  const float inv = lt > 0.0f ? (DROP ? p.keep_scale : 1.0f) / lt : 0.0f;
  if (qvalid) {
    const int64_t ob = b * p.q_sb + h * p.q_sh + qrow * p.q_st;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dd = d * 32 + 8 * i4 + 4 * g;
        if (OUT_BF16) {
          __bf16* op = (__bf16*)p.o + ob + dd;
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[d][4 * i4 + e] * inv);
          *(bf16x4*)op = v;
        } else {
          float* op = (float*)p.o + ob + dd;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[d][4 * i4 + e] * inv;
          *(f32x4*)op = v;
        }
      }
    if (p.lse && g == 0) p.lse[(b * p.Hq + h) * p.Tq + qrow] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

int mode_of(const FwdParams& p) {
  switch (p.bias) {
    case BIAS_NONE: return M_NONE;
    case BIAS_CAUSAL:
    case BIAS_SLIDING: return M_INDEX;
    case BIAS_ADDITIVE:
    case BIAS_BOOL: return M_TENSOR;
    case BIAS_RELPOS: return p.term_h ? M_RELPOS_ROW : M_RELPOS_FUSED;
    default: return -1;
  }
}

template <int D, int MODE>
hipError_t launch_mode(const FwdParams& p, hipStream_t s) {
  const int64_t grp = p.Hq / p.Hkv;
  const int hpw = (grp % 4 == 0) ? 4 : (grp % 2 == 0) ? 2 : 1;
  const int64_t rows = 32 * (4 / hpw);
  dim3 grid((unsigned)((p.Tq + rows - 1) / rows), (unsigned)(p.Hq / hpw), (unsigned)p.B);
  constexpr bool CAN_DROP = MODE == M_NONE || MODE == M_INDEX || MODE == M_TENSOR;
  if (CAN_DROP && p.keep) {
    if (p.out_dtype == 1) hipLaunchKernelGGL((flash_mfma_kernel<D, MODE, true, CAN_DROP>), grid, dim3(256), 0, s, p, hpw);
    else hipLaunchKernelGGL((flash_mfma_kernel<D, MODE, false, CAN_DROP>), grid, dim3(256), 0, s, p, hpw);
  } else if (p.out_dtype == 1) {
    hipLaunchKernelGGL((flash_mfma_kernel<D, MODE, true, false>), grid, dim3(256), 0, s, p, hpw);
  } else {
    hipLaunchKernelGGL((flash_mfma_kernel<D, MODE, false, false>), grid, dim3(256), 0, s, p, hpw);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t s) {
  switch (mode_of(p)) {
    case M_NONE: return launch_mode<D, M_NONE>(p, s);
    case M_INDEX: return launch_mode<D, M_INDEX>(p, s);
    case M_TENSOR: return launch_mode<D, M_TENSOR>(p, s);
    case M_RELPOS_ROW: return launch_mode<D, M_RELPOS_ROW>(p, s);
    case M_RELPOS_FUSED: return D == 64 ? launch_mode<64, M_RELPOS_FUSED>(p, s) : hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool relpos_fused_supported(const FwdParams& p) {
  return p.dtype == 1 && p.D == 64 && p.grid_w == 64 && p.grid_h >= 1 && p.grid_h <= 64 && p.rel_h && p.rel_w &&
         p.Tq == (int64_t)p.grid_h * 64 && p.Tkv == p.Tq;
}

bool flash_mfma_supports(const FwdParams& p) {
  if (p.dtype != 1 || (p.D != 64 && p.D != 128) || p.num_splits != 1) return false;
  if (mode_of(p) < 0) return false;
  if (p.bias == BIAS_RELPOS) {
    if (p.D != 64 || p.grid_w != 64) return false;
    if (!p.term_h && !relpos_fused_supported(p)) return false;
  }
  if (p.keep && p.bias == BIAS_RELPOS) return false;      // dropout runs with index / tensor masks only
  // Tensor masks index keys with 32-bit deltas inside a tile.
  if ((p.bias == BIAS_ADDITIVE || p.bias == BIAS_BOOL) && p.ms[3] * 4 * 64 > INT32_MAX) return false;
  return true;
}

hipError_t launch_flash_mfma(const FwdParams& p, hipStream_t s) {
  return p.D == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace sdpa
