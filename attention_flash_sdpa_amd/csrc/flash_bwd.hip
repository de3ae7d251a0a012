// Backward of fused attention on gfx950 matrix cores (MFMA 32x32x16, bf16 / fp16).
//
// For O = (W * Z) . V with W = softmax(scale * Q.K^T + B) and Z the dropout
// factor ([Axon PR 650] "Axon.Layers.scaled_dot_product_attention/4",
// description: attention-probability dropout in :train mode), the gradients
// of a loss with upstream gradient dO are
//   dV  = (W * Z)^T . dO
//   dW  = (dO . V^T) * Z
//   dS  = W * (dW - delta),   delta_i = sum_j W_ij dW_ij = dO_i . O_i
//   dQ  = scale * dS . K,     dK = scale * dS^T . Q
// The weights are rebuilt tile by tile from Q, K and the forward pass's row
// log-sum-exp (W = exp(s - lse)), so no T_q x T_kv array is stored.
//
// Three launches, none with atomics (the result is bitwise deterministic):
//   delta: rowsum(dO * O) per query row;
//   dK/dV: one workgroup per 128 keys (4 waves x 32 keys, K and V of the wave
//          held in registers), looping over the query heads that share the KV
//          head and over 64-query tiles of Q and dO staged through LDS;
//   dQ:    one workgroup per 128 query rows (4 waves x 32 rows, Q and dO in
//          registers), looping over 64-key tiles of K and V staged through LDS.
//
// Matrix-core layouts (32x32x16: A lane l holds row l % 32, k = 8 (l / 32) .. +7;
// B lane l holds column l % 32, same k; D lane l holds column l % 32, rows
// 8 (r / 4) + 4 (l / 32) + r % 4 for r = 0..15):
//   dK/dV: S[q, key] = Q . K^T and dW[q, key] = dO . V^T put one key per lane,
//          16 queries in registers.  Those registers are directly the B operand
//          of dV^T[d, key] += dO^T . (W*Z) and dK^T[d, key] += Q^T . dS over a
//          16-query chunk, the k index running over queries in the order the
//          D layout holds them; dO^T and Q^T come from the row-major LDS tiles
//          through the transposing LDS read (ds_read_b64_tr_b16), which reads
//          rows in exactly that order.
//   dQ:    S^T[key, q] = K . Q^T and dW^T = V . dO^T put one query per lane;
//          dQ^T[d, q] += K^T . dS^T with K^T from the K tile by transposing reads.
// Q, dO (dK/dV) and K (dQ) tiles are read both by 16-byte rows and by
// transposing reads, so their 16-byte chunks are XOR-swizzled with a pattern
// that keeps both kinds of access spread over the LDS banks.
#include "common.h"
#include "elem16.h"

#include <algorithm>
#include <mutex>

namespace sdpa {
namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.4426950408889634f;

// B_RELPOS64: rel-pos on a 64-wide grid, where a 64-key tile is one grid row.
enum BMode { B_NONE = 0, B_INDEX = 1, B_TENSOR = 2, B_RELPOS = 3, B_RELPOS64 = 4 };

// Rel-pos term rows held in LDS: grid_h + grid_w <= kMaxGT floats per query.
constexpr int kMaxGT = 128;

// Grid row and column of key `key` on a grid `gw` wide, from a known (row, col)
// of an earlier key `base` (key - base < 4 gw is enough for the short loop).
__device__ __forceinline__ void grid_step(int base_row, int base_col, int delta, int gw, int& row, int& col) {
  row = base_row;
  col = base_col + delta;
  while (col >= gw) {
    col -= gw;
    ++row;
  }
}

template <int D>
struct BCfg {
  static constexpr int PITCH = D * 2;   // bytes per LDS row (unpadded)
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int QC = D / 16;     // k-chunks of a contraction over head_dim
  static constexpr int DB = D / 32;     // 32-wide blocks of head_dim
  // Chunk c of row r sits at chunk position c ^ swz(r).  16 consecutive rows
  // read at one chunk index hit 16 distinct 16-byte bank groups.  A
  // transposing read takes 4 consecutive rows x 32 contiguous bytes for each
  // of two 16-column halves; the swizzle moves the 4 rows' pieces apart in
  // the bits above the lowest of the 32-byte group index, so the two halves
  // (whose group indices differ in the lowest bit) never share a group: 8
  // pieces in 8 distinct groups.  Depends on r % 16 only.
  static __device__ __forceinline__ int swz(int r) {
    if (D == 32) return (r >> 2) & 3;
    if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  }
};

template <typename E>
using V8 = typename Vec16<E>::x8;

template <typename E, int D>
__device__ __forceinline__ V8<E> ld_row(const lds_char* t, int row, int c, int g) {
  using C = BCfg<D>;
  return *(const __attribute__((address_space(3))) V8<E>*)(t + row * C::PITCH + (((2 * c + g) ^ C::swz(row)) << 4));
}

// A-operand fragment of the transposed tile: lane l gets column colbase + l % 32
// of rows rowbase + 4 (l / 32) + {0..3} and rowbase + 8 + 4 (l / 32) + {0..3}.
template <typename E, int D>
__device__ __forceinline__ V8<E> ld_tr(const lds_char* t, int rowbase, int colbase, int lane) {
  using C = BCfg<D>;
  const int j = lane & 15, dh = (lane >> 4) & 1, gg = lane >> 5;
  const int col = colbase + 16 * dh + 4 * (j & 3);
  const int r0 = rowbase + 4 * gg + (j >> 2), r1 = r0 + 8;
  const int chunk = col >> 3, within = (col & 7) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(t + r0 * C::PITCH + ((chunk ^ C::swz(r0)) << 4) + within));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(t + r1 * C::PITCH + ((chunk ^ C::swz(r1)) << 4) + within));
  const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V8<E>, a);
}

// The swizzle of row r depends only on r % 16, so every read below is the
// tile base + a compile-time row-group offset + a per-lane offset computed once.
template <int D>
struct LaneOff {
  int row[BCfg<D>::QC];                  // 16-byte row reads: row lane % 32, chunk 2 c + lane / 32
  int trlo[BCfg<D>::DB], trhi[BCfg<D>::DB];   // transposing reads of 16-row groups, column block nb
  __device__ __forceinline__ void init(int lane) {
    using C = BCfg<D>;
    const int nl = lane & 31, g = lane >> 5;
#pragma unroll
    for (int c = 0; c < C::QC; ++c) row[c] = nl * C::PITCH + (((2 * c + g) ^ C::swz(nl)) << 4);
    const int j = lane & 15, dh = (lane >> 4) & 1;
    const int r0 = 4 * g + (j >> 2), r1 = r0 + 8;
#pragma unroll
    for (int nb = 0; nb < C::DB; ++nb) {
      const int col = 32 * nb + 16 * dh + 4 * (j & 3);
      const int chunk = col >> 3, within = (col & 7) * 2;
      trlo[nb] = r0 * C::PITCH + ((chunk ^ C::swz(r0)) << 4) + within;
      trhi[nb] = r1 * C::PITCH + ((chunk ^ C::swz(r1)) << 4) + within;
    }
  }
};

// Row read of row base32 + lane % 32 (base32 a multiple of 32), chunk 2 c + lane / 32.
template <typename E, int D>
__device__ __forceinline__ V8<E> ld_row_o(const lds_char* t, int base32, const LaneOff<D>& lo, int c) {
  return *(const __attribute__((address_space(3))) V8<E>*)(t + base32 * BCfg<D>::PITCH + lo.row[c]);
}

// ld_tr for rowbase a multiple of 16 and colbase = 32 nb.
template <typename E, int D>
__device__ __forceinline__ V8<E> ld_tr_o(const lds_char* t, int rowbase, const LaneOff<D>& lo, int nb) {
  const lds_char* b = t + rowbase * BCfg<D>::PITCH;
  const s16x4 l4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(b + lo.trlo[nb]));
  const s16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(b + lo.trhi[nb]));
  const s16x8 a = __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V8<E>, a);
}

template <typename E>
__device__ __forceinline__ V8<E> pack8(const float* x) {
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, V8<E>);
}

template <typename T>
__device__ __forceinline__ T lds_load(const lds_char* p) {
  return *(const __attribute__((address_space(3))) T*)p;
}
template <typename T>
__device__ __forceinline__ void lds_store(lds_char* p, T v) {
  *(__attribute__((address_space(3))) T*)p = v;
}

// Workgroups are dealt to the 8 XCDs round-robin by linear id; renumber them so
// each XCD takes a contiguous range of (batch, head, block) and keeps those
// heads' tensors in its own L2.
__device__ __forceinline__ void xcd_block(int64_t& bx, int64_t& by, int64_t& bz) {
  const int64_t nblk = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int64_t lin = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t per = nblk / 8, rem = nblk % 8, xcd = lin % 8;
  const int64_t lid = xcd * per + min(xcd, rem) + lin / 8;
  bx = lid % gridDim.x;
  by = (lid / gridDim.x) % gridDim.y;
  bz = lid / ((int64_t)gridDim.x * gridDim.y);
}

__device__ __forceinline__ float mask_value(const BwdParams& p, int64_t b, int64_t h, int64_t i, int64_t j) {
  const int64_t off = b * p.ms[0] + h * p.ms[1] + i * p.ms[2] + j * p.ms[3];
  if (p.bias == BIAS_BOOL) return ((const uint8_t*)p.mdata)[off] ? 0.0f : -INFINITY;
  if (p.mdtype == 0) return ((const float*)p.mdata)[off];
  return (float)((const __bf16*)p.mdata)[off];
}

// lse in the log2 domain; a row with no allowed key (lse = -inf) or past the
// end gets +inf so that every weight of it is exp2(-inf) = 0.
__device__ __forceinline__ float lse2_of(const BwdParams& p, int64_t row, bool valid) {
  if (!valid) return INFINITY;
  const float l = p.lse[row];
  return l == -INFINITY ? INFINITY : l * kLog2e;
}

// Sum of the value held by lane l and lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float halves_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename G>
__device__ __forceinline__ void store4(G* dst, const float* v, float s) {
  if constexpr (sizeof(G) == 4) {
    *(f32x4*)dst = (f32x4){v[0] * s, v[1] * s, v[2] * s, v[3] * s};
  } else {
    typedef G g4 __attribute__((ext_vector_type(4)));
    *(g4*)dst = (g4){(G)(v[0] * s), (G)(v[1] * s), (G)(v[2] * s), (G)(v[3] * s)};
  }
}

// ------------------------------------------------------------------ delta --
template <typename E, typename EO, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p, int64_t rows) {
  constexpr int CH = D / 8;                // threads per row, 8 elements each
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / CH;
  const int c = (int)(gid % CH);
  float acc = 0.0f;
  if (row < rows) {
    const int64_t bh = row / p.Tq, i = row % p.Tq, b = bh / p.Hq, h = bh % p.Hq;
    const int64_t off = b * p.q_sb + h * p.q_sh + i * p.q_st + 8 * c;
    const V8<E> dv = *(const V8<E>*)((const E*)p.dout + off);
    float ov[8];
    if constexpr (sizeof(EO) == 4) {
      const f32x4 a = *(const f32x4*)((const float*)p.o + off);
      const f32x4 bq = *(const f32x4*)((const float*)p.o + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = a[e];
        ov[4 + e] = bq[e];
      }
    } else {
      const V8<E> o8 = *(const V8<E>*)((const E*)p.o + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = (float)o8[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)dv[e], ov[e], acc);
  }
#pragma unroll
  for (int m = 1; m < CH; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// ------------------------------------------------------------------ dK / dV --
template <typename E, int D, int MODE, bool DROP, typename G>
__global__ __launch_bounds__(256, (D == 128 ? 1 : 2)) void bwd_dkdv_kernel(BwdParams p) {
  using C = BCfg<D>;
  constexpr int BQ = 64;                           // queries per staged tile
  constexpr int TQ = BQ * C::PITCH;                // bytes of one Q or dO tile
  constexpr int NLD = BQ * C::CH / 256;            // 16-byte pieces per thread per tile
  constexpr int SOFF = 4 * TQ;                     // [buf][lse2 | delta][BQ] fp32
  constexpr int KOFF = SOFF + 2 * 2 * BQ * 4;      // [buf][wave][BQ] keep words
  // rel-pos: [buf][BQ][grid_h + grid_w] fp32 term rows; on a 64-wide grid only
  // the 64 columns and the two grid rows of the workgroup's keys: [buf][BQ][64], [BQ][2]
  constexpr int TOFF = KOFF + (DROP ? 2 * 4 * BQ * 4 : 0);
  // 64-wide grid: term_w transposed, [64 columns][BQ + 4 pad] (a lane's 4 consecutive queries
  // are one 16-byte read), then term_h at the 2 grid rows of the keys, [2][BQ]
  constexpr int TWQ = BQ + 4;
  constexpr int TBUF = MODE == B_RELPOS ? BQ * kMaxGT * 4 : (MODE == B_RELPOS64 ? (64 * TWQ + 2 * BQ) * 4 : 0);
  constexpr int SMEM = TOFF + 2 * TBUF;
  __shared__ __attribute__((aligned(16))) char smem_raw[SMEM];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, nl = lane & 31;
  int64_t bx, by, bz;
  xcd_block(bx, by, bz);
  const int64_t b = bz, hk = by;
  const int64_t kb0 = bx * 128;                    // first key of the workgroup
  const int64_t key = kb0 + 32 * wave + nl;        // this lane's key
  const bool kvalid = key < p.Tkv;
  const int grp = (int)(p.Hq / p.Hkv);
  const float c2 = p.scale * kLog2e;
  const int gh = p.grid_h, gw = p.grid_w, GT = gh + gw;
  const int jrow = MODE == B_RELPOS ? (int)((kvalid ? key : 0) / gw) : 0;   // this lane's key on the grid
  const int jcol = MODE == B_RELPOS ? (int)((kvalid ? key : 0) % gw) : 0;

  const E* kp = (const E*)p.k + b * p.k_sb + hk * p.k_sh;
  const E* vp = (const E*)p.v + b * p.k_sb + hk * p.k_sh;
  V8<E> kf[C::QC], vf[C::QC];
#pragma unroll
  for (int c = 0; c < C::QC; ++c) {
    kf[c] = kvalid ? *(const V8<E>*)(kp + key * p.k_st + 16 * c + 8 * g) : (V8<E>){};
    vf[c] = kvalid ? *(const V8<E>*)(vp + key * p.k_st + 16 * c + 8 * g) : (V8<E>){};
  }

  LaneOff<D> lo;
  lo.init(lane);

  // Queries that can see any key of the workgroup.
  int64_t qlo = 0, qhi = p.Tq;
  if (MODE == B_INDEX) {
    const int64_t klast = min(kb0 + 127, p.Tkv - 1);
    qlo = max((int64_t)0, kb0 - p.offset);
    if (p.bias == BIAS_SLIDING) qhi = min(p.Tq, klast - p.offset + p.window);
  }
  const int64_t qt0 = qlo / BQ;
  const int nqt = qhi > qlo ? (int)((qhi + BQ - 1) / BQ - qt0) : 0;
  const int niter = nqt * grp;

  V8<E> qst[NLD], dst_[NLD];
  float sval = 0.0f;
  uint32_t kwv = 0;
  auto gload = [&](int it) {
    const int64_t hq = hk * grp + it / nqt;
    const int64_t q0 = (qt0 + it % nqt) * BQ;
    const E* qb = (const E*)p.q + b * p.q_sb + hq * p.q_sh;
    const E* db = (const E*)p.dout + b * p.q_sb + hq * p.q_sh;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 256 * u, row = idx / C::CH, ch = idx % C::CH;
      const bool ok = q0 + row < p.Tq;
      qst[u] = ok ? *(const V8<E>*)(qb + (q0 + row) * p.q_st + 8 * ch) : (V8<E>){};
      dst_[u] = ok ? *(const V8<E>*)(db + (q0 + row) * p.q_st + 8 * ch) : (V8<E>){};
    }
    const int64_t rbase = (b * p.Hq + hq) * p.Tq;
    if (tid < BQ) {
      sval = lse2_of(p, rbase + q0 + tid, q0 + tid < p.Tq);
    } else if (tid < 2 * BQ) {
      const int64_t qi = q0 + tid - BQ;
      sval = qi < p.Tq ? p.delta[rbase + qi] : 0.0f;
    }
    if (DROP) {
      const int64_t qi = q0 + (tid & 63);
      const int64_t w = kb0 / 32 + (tid >> 6);
      kwv = (qi < p.Tq && w < p.keep_words) ? p.keep[(rbase + qi) * p.keep_words + w] : 0u;
    }
  };
  auto lstore = [&](int buf, int it) {
    lds_char* qt = smem + buf * 2 * TQ;
    lds_char* dt = qt + TQ;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 256 * u, row = idx / C::CH, ch = idx % C::CH;
      const int off = row * C::PITCH + ((ch ^ C::swz(row)) << 4);
      lds_store(qt + off, qst[u]);
      lds_store(dt + off, dst_[u]);
    }
    if (tid < 2 * BQ) lds_store(smem + SOFF + buf * 2 * BQ * 4 + tid * 4, sval);
    if (DROP) lds_store(smem + KOFF + buf * 4 * BQ * 4 + tid * 4, kwv);
    if (MODE == B_RELPOS) {          // term rows of the tile's queries: [q][term_h row | term_w row]
      const int64_t hq = hk * grp + it / nqt;
      const int64_t q0 = (qt0 + it % nqt) * BQ;
      const int64_t rbase = (b * p.Hq + hq) * p.Tq;
      lds_char* tl = smem + TOFF + buf * TBUF;
      for (int e0 = 0; e0 < BQ * GT; e0 += 6 * 256) {    // 6 loads in flight per lane, then the stores
        float v[6];
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const int e = e0 + tid + 256 * u, q = e / GT, c = e % GT;
          v[u] = 0.0f;
          if (e < BQ * GT && q0 + q < p.Tq)
            v[u] = c < gh ? p.term_h[(rbase + q0 + q) * gh + c] : p.term_w[(rbase + q0 + q) * gw + c - gh];
        }
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const int e = e0 + tid + 256 * u;
          if (e < BQ * GT) lds_store(tl + e * 4, v[u]);
        }
      }
    }
    if (MODE == B_RELPOS64) {
      // [q][64] term_w rows (one contiguous 16 KB range: four 16-byte loads per
      // thread, all in flight), then [q][2] term_h at the 2 grid rows of the keys
      const int64_t hq = hk * grp + it / nqt;
      const int64_t q0 = (qt0 + it % nqt) * BQ;
      const int64_t rbase = (b * p.Hq + hq) * p.Tq;
      const int64_t row0 = kb0 / 64;
      lds_char* tl = smem + TOFF + buf * TBUF;
      const float* src = p.term_w + (rbase + q0) * 64;
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 4 * (tid + 256 * u);              // float index in the [64][64] block
        v[u] = (q0 + e / 64 < p.Tq) ? *(const f32x4*)(src + e) : (f32x4){};
      }
      float hv = 0.0f;
      if (tid < 2 * BQ) {
        const int q = tid >> 1, c = tid & 1;
        if (q0 + q < p.Tq && row0 + c < gh) hv = p.term_h[(rbase + q0 + q) * gh + row0 + c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {                     // transposed: [column][query]
        const int e = 4 * (tid + 256 * u), q = e / 64, c = e % 64;
#pragma unroll
        for (int x = 0; x < 4; ++x) lds_store(tl + ((c + x) * TWQ + q) * 4, v[u][x]);
      }
      if (tid < 2 * BQ) lds_store(tl + (64 * TWQ + (tid & 1) * BQ + (tid >> 1)) * 4, hv);
    }
  };

  f32x16_e dvT[C::DB], dkT[C::DB];
#pragma unroll
  for (int nb = 0; nb < C::DB; ++nb) {
    dvT[nb] = (f32x16_e){};
    dkT[nb] = (f32x16_e){};
  }
  if (niter > 0) {
    gload(0);
    lstore(0, 0);
  }
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < niter;
    if (more) gload(it + 1);
    const int64_t hq = hk * grp + it / nqt;
    const int64_t q0 = (qt0 + it % nqt) * BQ;
    const lds_char* qt = smem + buf * 2 * TQ;
    const lds_char* dt = qt + TQ;
    const lds_char* l2s = smem + SOFF + buf * 2 * BQ * 4;
    const lds_char* dls = l2s + BQ * 4;
    const lds_char* kws = smem + KOFF + buf * 4 * BQ * 4 + wave * BQ * 4;
    const lds_char* tls = smem + TOFF + buf * TBUF;
#pragma unroll 1
    for (int s = 0; s < 2; ++s) {
      const int64_t qa = q0 + 32 * s;
      if (qa >= p.Tq) break;
      // Index masks: skip a sub-tile with no allowed (query, key) pair, test per score
      // only where the band edge crosses it (allowed: key - offset <= q < key - offset + window).
      bool edge = false;
      int qa32 = 0, mlo = 0, mhi = 0;
      if (MODE == B_INDEX) {
        const int64_t kw0 = kb0 + 32 * wave;
        if (kw0 > qa + 31 + p.offset) continue;
        const bool sl = p.bias == BIAS_SLIDING;
        if (sl && kw0 + 31 <= qa + p.offset - p.window) continue;
        edge = !(kw0 + 31 <= qa + p.offset && (!sl || kw0 > qa + 31 + p.offset - p.window));
        const int64_t l64 = key - p.offset, h64 = sl ? key - p.offset + p.window : p.Tq + 64;
        qa32 = (int)qa;
        mlo = (int)max(min(l64, (int64_t)INT32_MAX), (int64_t)INT32_MIN);
        mhi = (int)max(min(h64, (int64_t)INT32_MAX), (int64_t)INT32_MIN);
      }
      f32x16_e sacc = (f32x16_e){}, dpacc = (f32x16_e){};
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        sacc = mfma32(ld_row_o<E, D>(qt, 32 * s, lo, c), kf[c], sacc);
        dpacc = mfma32(ld_row_o<E, D>(dt, 32 * s, lo, c), vf[c], dpacc);
      }
      float l2[16], dl[16], pt[16], ds[16];
      uint32_t kw[16];
      f32x4 bias4 = (f32x4){};
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int qo = 32 * s + 8 * a + 4 * g;
        const f32x4 x = lds_load<f32x4>(l2s + qo * 4);
        const f32x4 y = lds_load<f32x4>(dls + qo * 4);
        u32x4 z = (u32x4){};
        if (DROP) z = lds_load<u32x4>(kws + qo * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l2[4 * a + e] = x[e];
          dl[4 * a + e] = y[e];
          kw[4 * a + e] = z[e];
        }
      }
      // exponent arguments first, then the index mask under one wave-uniform branch, then
      // the exponentials: masked scores become -inf before exp2 (exp2(-inf) = 0), so no
      // score takes a branch of its own
      float xs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t qq = qa + 8 * (r / 4) + 4 * g + (r % 4);
        float xb = -l2[r];
        if (MODE == B_TENSOR) {
          if (kvalid && qq < p.Tq) xb += mask_value(p, b, hq, qq, key) * kLog2e;
        }
        if (MODE == B_RELPOS) {      // term_h[q, row(key)] + term_w[q, col(key)] from the staged rows
          const int qo = 32 * s + 8 * (r / 4) + 4 * g + (r % 4);
          const float th = lds_load<float>(tls + (qo * GT + jrow) * 4);
          const float tw = lds_load<float>(tls + (qo * GT + gh + jcol) * 4);
          xb += (th + tw) * kLog2e;
        }
        if (MODE == B_RELPOS64) {    // the wave's keys lie in grid row kb0 / 64 + wave / 2
          if (r % 4 == 0) {           // term_h + term_w of the 4 queries 32 s + 8 (r / 4) + 4 g + 0..3
            const int qo0 = 32 * s + 8 * (r / 4) + 4 * g;
            const f32x4 tw4 = lds_load<f32x4>(tls + ((32 * (wave & 1) + nl) * TWQ + qo0) * 4);
            const f32x4 th4 = lds_load<f32x4>(tls + (64 * TWQ + (wave >> 1) * BQ + qo0) * 4);
            bias4 = (tw4 + th4) * kLog2e;
          }
          xb += bias4[r % 4];
        }
        // A lane is a key: past the end of the keys (zero K, V rows, finite scores; on
        // 64-wide grids the staged term rows of such keys are zero) its weights only reach
        // this key's own dK / dV columns, which are not stored, so no select is needed.
        if (MODE == B_NONE || MODE == B_INDEX || MODE == B_RELPOS64) xs[r] = fmaf(sacc[r], c2, xb);
        else xs[r] = kvalid ? fmaf(sacc[r], c2, xb) : -INFINITY;
      }
      if (MODE == B_INDEX && edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q32 = qa32 + 8 * (r / 4) + 4 * g + (r % 4);
          xs[r] = ((q32 >= mlo) & (q32 < mhi)) ? xs[r] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(xs[r]);
        float dw = dpacc[r];
        if (DROP) {
          const bool kept = (kw[r] >> nl) & 1u;
          pt[r] = kept ? pr * p.keep_scale : 0.0f;
          dw = kept ? dw * p.keep_scale : 0.0f;
        } else {
          pt[r] = pr;
        }
        ds[r] = pr * (dw - dl[r]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const V8<E> pb = pack8<E>(pt + 8 * c);
        const V8<E> sb = pack8<E>(ds + 8 * c);
#pragma unroll
        for (int nb = 0; nb < C::DB; ++nb) {
          dvT[nb] = mfma32(ld_tr_o<E, D>(dt, 32 * s + 16 * c, lo, nb), pb, dvT[nb]);
          dkT[nb] = mfma32(ld_tr_o<E, D>(qt, 32 * s + 16 * c, lo, nb), sb, dkT[nb]);
        }
      }
    }
    if (more) lstore(buf ^ 1, it + 1);
    __syncthreads();
  }

  // dV^T / dK^T: lane = key, registers = head dims 32 nb + 8 (r / 4) + 4 g + r % 4.
  if (kvalid) {
    G* dkp = (G*)p.dk + b * p.k_sb + hk * p.k_sh + key * p.k_st;
    G* dvp = (G*)p.dv + b * p.k_sb + hk * p.k_sh + key * p.k_st;
#pragma unroll
    for (int nb = 0; nb < C::DB; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * nb + 8 * i4 + 4 * g;
        float a[4], c4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dvT[nb][4 * i4 + e];
          c4[e] = dkT[nb][4 * i4 + e];
        }
        store4(dvp + d, a, 1.0f);
        store4(dkp + d, c4, p.scale);
      }
  }
}

// ---------------------------------------------------------------------- dQ --
// RPS (rel-pos grids of at most 32 x 32): the per-query sums of dS over grid rows and
// columns are matrix products, dT_h^T = E_h^T . dS^T with E_h[key][y] = 1 iff key lies in
// grid row y (E_w alike), fed the same packed dS as the dQ product; no LDS sums.
// Two waves per SIMD, also at head_dim 128 with no mask or an index mask and
// no dropout (the dQ accumulator, Q and dO fragments fit 256 registers with a
// few spills; the second wave hides the per-tile latencies: gqa_causal
// backward 3.06 -> 2.82 ms); the other head_dim-128 instances need more.
template <typename E, int D, int MODE, bool DROP, typename G, bool RPS = false>
__global__ __launch_bounds__(256, (D == 128 && (DROP || !(MODE == B_NONE || MODE == B_INDEX)) ? 1 : 2))
void bwd_dq_kernel(BwdParams p) {
  using C = BCfg<D>;
  constexpr int BN = 64;                           // keys per staged tile
  constexpr int TK = BN * C::PITCH;
  constexpr int NLD = BN * C::CH / 256;
  // [buf][K | V] tiles; rel-pos: then the per-query sums of dS, [128 q][grid_h + grid_w] fp32;
  // 64-wide grid: then term_w of the workgroup's 128 queries, [128 q][64 + 4 pad] fp32
  constexpr int DOFF = 4 * TK;
  constexpr int TWP = 68;
  __shared__ __attribute__((aligned(16))) char smem_raw[DOFF + (MODE == B_RELPOS && !RPS ? 128 * kMaxGT * 4 : 0) +
                                                       (MODE == B_RELPOS64 ? 128 * TWP * 4 : 0)];
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, nl = lane & 31;
  int64_t bx, by, bz;
  xcd_block(bx, by, bz);
  const int64_t b = bz, h = by;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t wg_q0 = bx * 128;
  const int64_t wq0 = wg_q0 + 32 * wave;
  const int64_t qrow = wq0 + nl;
  const bool qvalid = qrow < p.Tq;
  const float c2 = p.scale * kLog2e;

  const int64_t qoff = b * p.q_sb + h * p.q_sh + (qvalid ? qrow : 0) * p.q_st;
  V8<E> qf[C::QC], of[C::QC];
#pragma unroll
  for (int c = 0; c < C::QC; ++c) {
    qf[c] = qvalid ? *(const V8<E>*)((const E*)p.q + qoff + 16 * c + 8 * g) : (V8<E>){};
    of[c] = qvalid ? *(const V8<E>*)((const E*)p.dout + qoff + 16 * c + 8 * g) : (V8<E>){};
  }
  const int64_t srow = (b * p.Hq + h) * p.Tq + qrow;
  const float l2 = lse2_of(p, srow, qvalid);
  const float dl = qvalid ? p.delta[srow] : 0.0f;

  int64_t lo = 0, hi = p.Tkv;
  if (MODE == B_INDEX) {
    const int64_t wg_q1 = min(wg_q0 + 127, p.Tq - 1);
    hi = min(hi, wg_q1 + p.offset + 1);
    if (p.bias == BIAS_SLIDING) lo = max((int64_t)0, wg_q0 + p.offset - p.window + 1);
  }
  const int64_t t0 = lo / BN;
  const int ntiles = hi > lo ? (int)((hi - t0 * BN + BN - 1) / BN) : 0;

  const int gh = p.grid_h, gw = p.grid_w, GT = gh + gw;
  const float* thr = nullptr;
  const float* twr = nullptr;
  __attribute__((address_space(3))) float* dts = nullptr;
  constexpr bool FASTM = MODE == B_NONE || MODE == B_INDEX || MODE == B_RELPOS64;
  // the accumulators are read after the loop behind lane-divergent branches on
  // the rel-pos paths (not needed on the matrix-product path at head_dim 32 / 64)
  constexpr bool FENCE_END = !(RPS && D != 128);
  const bool sl = MODE == B_INDEX && p.bias == BIAS_SLIDING;
  // 64-wide grid: a 64-key tile is one grid row y, and the lane's 32 registers of
  // a tile always hold the same 32 columns, so the running sums of dS per column
  // stay in registers (term_w of those columns is re-read per tile, from cache).
  constexpr bool RP64 = MODE == B_RELPOS64;
  float dtw[RP64 ? 2 : 1][16];
  // term_w rows staged in LDS (read once per tile from there); rows padded by 16 bytes
  const lds_char* twq = smem + DOFF + (32 * wave + nl) * TWP * 4;
  if (RP64) {
    const float* src = p.term_w + ((b * p.Hq + h) * p.Tq + wg_q0) * 64;
    for (int e = tid; e < 128 * 16; e += 256) {      // 16-byte pieces of the [128][64] block
      const int q = e >> 4, c4 = (e & 15) * 4;
      const f32x4 v = wg_q0 + q < p.Tq ? *(const f32x4*)(src + q * 64 + c4) : (f32x4){};
      lds_store(smem + DOFF + (q * TWP + c4) * 4, v);
    }
  }
  if (RP64) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dtw[kb][r] = 0.0f;
  }
  if (RP64) thr = p.term_h + (qvalid ? srow : 0) * gh;
  if (MODE == B_RELPOS) {
    thr = p.term_h + (qvalid ? srow : 0) * gh;
    twr = p.term_w + (qvalid ? srow : 0) * gw;
  }
  f32x16_e dthT = (f32x16_e){}, dtwT = (f32x16_e){};    // RPS: rows y / x of this lane's query
  if (MODE == B_RELPOS && !RPS) {
    dts = (__attribute__((address_space(3))) float*)(smem + DOFF);
    for (int e = tid; e < 128 * GT; e += 256) dts[e] = 0.0f;
    dts += (32 * wave + nl) * GT;     // this lane's query row
  }

  const E* kp = (const E*)p.k + b * p.k_sb + hk * p.k_sh;
  const E* vp = (const E*)p.v + b * p.k_sb + hk * p.k_sh;
  V8<E> kst[NLD], vst[NLD];
  auto gload = [&](int it) {
    const int64_t k0 = (t0 + it) * BN;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 256 * u, row = idx / C::CH, ch = idx % C::CH;
      const bool ok = k0 + row < p.Tkv;
      kst[u] = ok ? *(const V8<E>*)(kp + (k0 + row) * p.k_st + 8 * ch) : (V8<E>){};
      vst[u] = ok ? *(const V8<E>*)(vp + (k0 + row) * p.k_st + 8 * ch) : (V8<E>){};
    }
  };
  auto lstore = [&](int buf) {
    lds_char* ks = smem + buf * 2 * TK;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 256 * u, row = idx / C::CH, ch = idx % C::CH;
      const int off = row * C::PITCH + ((ch ^ C::swz(row)) << 4);
      lds_store(ks + off, kst[u]);
      lds_store(ks + TK + off, vst[u]);
    }
  };

  f32x16_e dqT[C::DB];
#pragma unroll
  for (int nb = 0; nb < C::DB; ++nb) dqT[nb] = (f32x16_e){};
  float th_next = (RP64 && qvalid && ntiles > 0) ? thr[t0] : 0.0f;   // 64-wide grid: term_h of the first tile's row
  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) gload(it + 1);
    const int64_t k0 = (t0 + it) * BN;
    const lds_char* ks = smem + buf * 2 * TK;
    const lds_char* vs = ks + TK;
    bool skip = wq0 >= p.Tq;
    if (MODE == B_INDEX) {
      if (k0 > wq0 + 31 + p.offset) skip = true;
      if (p.bias == BIAS_SLIDING && k0 + BN - 1 <= wq0 + p.offset - p.window) skip = true;
    }
    if (!skip) {
      uint32_t kw[2] = {0u, 0u};
      if (DROP && qvalid) {
        const int64_t w0 = k0 / 32;
        const uint32_t* kr = p.keep + srow * p.keep_words;
        kw[0] = kr[w0];
        kw[1] = w0 + 1 < p.keep_words ? kr[w0 + 1] : 0u;
      }
      // 64-wide grid: term_h of this tile's grid row, and the row's running dS sum
      const float th2 = RP64 ? th_next * kLog2e : 0.0f;
      if (RP64 && it + 1 < ntiles) th_next = qvalid ? thr[k0 / 64 + 1] : 0.0f;   // next tile's grid row
      float tsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // No mask, index masks, 64-wide rel-pos grids: masks are tested only on the
        // 32-key sub-tiles that the band edge or the end of the keys crosses (a
        // wave-uniform test), per score in 32-bit offsets from the sub-tile's first
        // key (allowed: lim_lo < offset <= lim_hi); sub-tiles with no allowed pair
        // for the wave's queries are skipped.
        const int64_t kbase = k0 + 32 * kb;
        bool edge = false;
        int lim_hi = 31, lim_lo = -1;
        if (FASTM) {
          if (MODE == B_INDEX) {
            if (kbase > wq0 + 31 + p.offset) continue;
            if (sl && kbase + 31 <= wq0 + p.offset - p.window) continue;
            if (kbase + 31 > wq0 + p.offset) edge = true;
            if (sl && kbase <= wq0 + 31 + p.offset - p.window) edge = true;
          }
          if (kbase + 32 > p.Tkv) edge = true;
          if (edge) {
            int64_t h64 = p.Tkv - 1 - kbase, l64 = -1;
            if (MODE == B_INDEX) {
              h64 = min(h64, qrow + p.offset - kbase);
              if (sl) l64 = qrow + p.offset - p.window - kbase;
            }
            lim_hi = (int)max(min(h64, (int64_t)31), (int64_t)-1);
            lim_lo = (int)max(min(l64, (int64_t)32), (int64_t)-1);
          }
        }
        f32x16_e sacc = (f32x16_e){}, dpacc = (f32x16_e){};
#pragma unroll
        for (int c = 0; c < C::QC; ++c) {
          sacc = mfma32(ld_row<E, D>(ks, 32 * kb + nl, c, g), qf[c], sacc);
          dpacc = mfma32(ld_row<E, D>(vs, 32 * kb + nl, c, g), of[c], dpacc);
        }
        // The mask / term reads below branch on lane conditions before sacc and
        // dpacc are read: fence them.  Not on the matrix-product dS-sum path at
        // head_dim 32 / 64, where the compiler's own wait states hold on every
        // path (tests/test_isa_hazards.py checks each instance) and the fence's
        // AGPR operands would force copies and spills.
        constexpr bool FENCE = !FASTM && !(MODE == B_RELPOS && RPS && D != 128);
        if (FENCE) mfma_drain(sacc, dpacc);
        float ds[16];
        // rel-pos: grid (row, col) of the first key of each group of 4 this lane holds
        int grow[4] = {0, 0, 0, 0}, gcol[4] = {0, 0, 0, 0};
        if (MODE == B_RELPOS) {
          const int64_t kbase = k0 + 32 * kb;
          const int brow = (int)(kbase / gw), bcol = (int)(kbase % gw);
#pragma unroll
          for (int a = 0; a < 4; ++a) grid_step(brow, bcol, 8 * a + 4 * g, gw, grow[a], gcol[a]);
        }
        int krow[16], kcol[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (MODE == B_RELPOS) grid_step(grow[r / 4], gcol[r / 4], r % 4, gw, krow[r], kcol[r]);
          else krow[r] = kcol[r] = 0;
        }
        float tw2[RP64 ? 16 : 1];
        if (RP64) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const f32x4 t = lds_load<f32x4>(twq + (32 * kb + 8 * a + 4 * g) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) tw2[4 * a + e] = t[e] * kLog2e;
          }
        }
        if (FASTM) {
          float xs[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float xb = -l2;
            if (RP64) xb += th2 + tw2[r];
            xs[r] = fmaf(sacc[r], c2, xb);
          }
          if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kofs = 8 * (r / 4) + 4 * g + (r % 4);
              xs[r] = ((kofs <= lim_hi) & (kofs > lim_lo)) ? xs[r] : -INFINITY;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kofs = 8 * (r / 4) + 4 * g + (r % 4);
            const float pr = __builtin_amdgcn_exp2f(xs[r]);      // exp2(-inf) = 0: masked scores
            float dw = dpacc[r];
            if (DROP) dw = ((kw[kb] >> kofs) & 1u) ? dw * p.keep_scale : 0.0f;
            ds[r] = pr * (dw - dl);
          }
        }
#pragma unroll
        for (int r = 0; r < 16 && !FASTM; ++r) {
          const int kofs = 8 * (r / 4) + 4 * g + (r % 4);
          const int64_t key = k0 + 32 * kb + kofs;
          bool ok = key < p.Tkv;
          float xb = -l2;
          if (MODE == B_RELPOS) {
            if (ok && qvalid) xb += (thr[krow[r]] + twr[kcol[r]]) * kLog2e;
          }
          if (RP64) xb += th2 + tw2[r];
          if (MODE == B_INDEX) {
            ok = ok && key <= qrow + p.offset;
            if (p.bias == BIAS_SLIDING) ok = ok && key > qrow + p.offset - p.window;
          }
          if (MODE == B_TENSOR) {
            if (ok && qvalid) xb += mask_value(p, b, h, qrow, key) * kLog2e;
          }
          const float pr = ok ? __builtin_amdgcn_exp2f(fmaf(sacc[r], c2, xb)) : 0.0f;
          float dw = dpacc[r];
          if (DROP) dw = ((kw[kb] >> kofs) & 1u) ? dw * p.keep_scale : 0.0f;
          ds[r] = pr * (dw - dl);
        }
        if (RP64) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            dtw[kb][r] += ds[r];
            tsum += ds[r];
          }
        }
        if (MODE == B_RELPOS && !RPS) {
          // dterm_h[q, row] and dterm_w[q, col] collect dS.  Lanes l and l + 32 hold the
          // same query (keys 8 (r / 4) + r % 4 and 4 further on), so they swap their dS:
          // then both hold all 32 keys of the sub-tile, lane half 0 adds every key into
          // the grid-row sums [0, gh) of the query's LDS row and lane half 1 into the
          // grid-column sums [gh, gh + gw).  Each LDS word has one writer lane, and that
          // lane adds in a fixed order.
          const int64_t kb0 = k0 + 32 * kb;
          const int brow = (int)(kb0 / gw), bcol = (int)(kb0 % gw);
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            int r0, c0, r1, c1;
            grid_step(brow, bcol, 8 * a, gw, r0, c0);         // keys of lane half 0
            grid_step(brow, bcol, 8 * a + 4, gw, r1, c1);     // keys of lane half 1
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * a + e;
              auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ds[r]), __float_as_uint(ds[r]), false, false);
              const float v0 = __uint_as_float(sw[0]), v1 = __uint_as_float(sw[1]);   // half 0's, half 1's dS
              int y0, x0, y1, x1;
              grid_step(r0, c0, e, gw, y0, x0);
              grid_step(r1, c1, e, gw, y1, x1);
              const bool in0 = kb0 + 8 * a + e < p.Tkv, in1 = kb0 + 8 * a + 4 + e < p.Tkv;
              if (qvalid) {
                if (in0) dts[g ? gh + x0 : y0] += v0;
                if (in1) dts[g ? gh + x1 : y1] += v1;
              }
            }
          }
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const V8<E> sb = pack8<E>(ds + 8 * c);
#pragma unroll
          for (int nb = 0; nb < C::DB; ++nb)
            dqT[nb] = mfma32(ld_tr<E, D>(ks, 32 * kb + 16 * c, 32 * nb, lane), sb, dqT[nb]);
          if (RPS) {
            // element e of this lane's k-slice is key offset 8 (r / 4) + 4 g + r % 4, r = 8 c + e
            // (the order dS is packed in); A row = lane % 32 is the grid row / column index
            float eh[8], ew[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              eh[e] = krow[8 * c + e] == nl ? 1.0f : 0.0f;
              ew[e] = kcol[8 * c + e] == nl ? 1.0f : 0.0f;
            }
            dthT = mfma32(pack8<E>(eh), sb, dthT);
            dtwT = mfma32(pack8<E>(ew), sb, dtwT);
          }
        }
      }
      if (RP64) {
        const float tot = halves_sum(tsum);      // the two lane halves hold the row's other keys
        if (g == 0 && qvalid) p.dterm_h[srow * gh + k0 / 64] = tot;
      }
    }
    if (more) lstore(buf ^ 1);
    // The rel-pos paths read the accumulators after the loop behind
    // lane-divergent branches: fence them there.  (Elsewhere the compiler's own
    // wait states hold on every path, and an AGPR fence on the VGPR-resident
    // accumulators would only add copies and spills.)
    if (MODE == B_RELPOS && FENCE_END && !more) {
#pragma unroll
      for (int nb = 0; nb < C::DB; ++nb) mfma_drain(dqT[nb]);
      if (RPS) mfma_drain(dthT, dtwT);
    }
    __syncthreads();
  }

  if (MODE == B_RELPOS || RP64) {
    // scale * dS . K in fp32 (the tables' part is added by the tail kernel) and the
    // per-query dS sums (each lane half writes every other entry of its query row)
    __syncthreads();
    if (qvalid) {
      float* acc = p.dq_acc + srow * p.D;
#pragma unroll
      for (int nb = 0; nb < C::DB; ++nb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float a[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] = dqT[nb][4 * i4 + e];
          store4(acc + 32 * nb + 8 * i4 + 4 * g, a, p.scale);
        }
      if (RP64) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            store4(p.dterm_w + srow * 64 + 32 * kb + 8 * a + 4 * g, &dtw[kb][4 * a], 1.0f);
      } else if (RPS) {
        // lane = query; rows y = 8 (r / 4) + 4 g + r % 4 of the two products
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int y = 8 * (r / 4) + 4 * g + (r % 4);
          if (y < gh) p.dterm_h[srow * gh + y] = dthT[r];
          if (y < gw) p.dterm_w[srow * gw + y] = dtwT[r];
        }
      } else {
        for (int c = g; c < GT; c += 2) {
          const float v = dts[c];
          if (c < gh) p.dterm_h[srow * gh + c] = v;
          else p.dterm_w[srow * gw + c - gh] = v;
        }
      }
    }
    return;
  }
  // dQ^T: lane = query, registers = head dims 32 nb + 8 (r / 4) + 4 g + r % 4.
  if (qvalid) {
    G* dqp = (G*)p.dq + qoff;
#pragma unroll
    for (int nb = 0; nb < C::DB; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = dqT[nb][4 * i4 + e];
        store4(dqp + 32 * nb + 8 * i4 + 4 * g, a, p.scale);
      }
  }
}

// ---------------------------------------------------------------- launchers --
int bmode_of(const BwdParams& p) {
  switch (p.bias) {
    case BIAS_NONE: return B_NONE;
    case BIAS_CAUSAL:
    case BIAS_SLIDING: return B_INDEX;
    case BIAS_ADDITIVE:
    case BIAS_BOOL: return B_TENSOR;
    case BIAS_RELPOS: return p.grid_w == 64 ? B_RELPOS64 : B_RELPOS;
    default: return -1;
  }
}

// The second stream of the current device for the dQ kernel (created on first
// use, default priority, not synchronising with the null stream) and the
// device's compute-unit count; a null stream when none is available, when
// the caller's stream belongs to another device than the current one, or
// when it is being captured into a graph (such calls keep every kernel on
// the caller's stream).
struct SideStream {
  hipStream_t stream;
  int cus;
};

SideStream side_stream(hipStream_t caller) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static SideStream per_dev[kMaxDevices] = {};
  int dev = 0, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return {nullptr, 0};
  if (hipStreamGetDevice(caller, &sdev) != hipSuccess || sdev != dev) return {nullptr, 0};
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return {nullptr, 0};
  std::lock_guard<std::mutex> lock(mu);
  SideStream& d = per_dev[dev];
  if (!d.stream) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return {nullptr, 0};
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return {nullptr, 0};
    d = {st, cus};
  }
  return d;
}

// dK/dV and dQ, then two tails that need dq: `tail` on the caller's stream
// and `side_tail`, independent of `tail`'s outputs (either may be null).
// The two kernels read the same inputs and delta and write disjoint
// outputs, so with p.concurrent the dQ kernel can run on the device's
// second stream beside the dK/dV kernel: the workgroups of each then fill
// CUs the other leaves idle.  That pays when a kernel's grid leaves at least
// a tenth of the workgroup slots of its last round empty (rounds of the
// workgroups the chip holds at once: SAM ViT-B global attention runs 384
// workgroups per kernel and batch item where 512 fit, its 14x14 windows 600
// per 25 windows).  Grids that fill their rounds (gqa_causal: 1024 and 4096
// workgroups, 256 at a time) run one after the other, which keeps each
// kernel's workgroups together in the caches.  Side by side, an event forks the second stream from the caller's
// after delta; `side_tail` follows dQ there, while `tail` runs on the
// caller's stream once dQ (a second event) and dK/dV are done, and a third
// event joins the second stream back, so work queued later on the caller's
// stream sees every output.  Returns the first HIP error.
template <typename E, int D, int MODE, bool DROP, typename G, bool RPS = false>
hipError_t launch_main(const BwdParams& p, hipStream_t s, BwdTail tail, BwdTail side_tail) {
  dim3 gkv((unsigned)((p.Tkv + 127) / 128), (unsigned)p.Hkv, (unsigned)p.B);
  dim3 gq((unsigned)((p.Tq + 127) / 128), (unsigned)p.Hq, (unsigned)p.B);
  hipStream_t side = nullptr;
  if (p.concurrent) {
    const SideStream ss = side_stream(s);
    const int64_t resident = (int64_t)ss.cus * (D == 128 ? 1 : 2);       // workgroups per CU at these launch bounds
    // fraction of the last round of resident workgroups a kernel leaves empty
    auto idle = [&](int64_t n) {
      const int64_t r = (n + resident - 1) / resident;
      return (double)(r * resident - n) / (double)(r * resident);
    };
    const int64_t nkv = (int64_t)gkv.x * gkv.y * gkv.z, nq = (int64_t)gq.x * gq.y * gq.z;
    if (ss.stream && resident > 0 && std::max(idle(nkv), idle(nq)) >= 0.1) side = ss.stream;
  }
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};        // fork, dq done, join
  for (int i = 0; side && i < 3; ++i) {
    if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      side = nullptr;
    }
  }
  if (side) {
    hipError_t e = hipEventRecord(ev[0], s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, ev[0], 0);
    if (e != hipSuccess) {                 // nothing launched yet: run everything on the caller's stream
      for (hipEvent_t x : ev) (void)hipEventDestroy(x);
      side = nullptr;
    }
  }
  if (!side) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, MODE, DROP, G>), gkv, dim3(256), 0, s, p);
    hipLaunchKernelGGL((bwd_dq_kernel<E, D, MODE, DROP, G, RPS>), gq, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && tail) e = tail(p, s);
    if (e == hipSuccess && side_tail) e = side_tail(p, s);
    return e;
  }
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, MODE, DROP, G, RPS>), gq, dim3(256), 0, side, p);
  hipError_t e = hipGetLastError();
  auto keep = [&e](hipError_t x) { if (e == hipSuccess) e = x; };
  keep(hipEventRecord(ev[1], side));
  if (e == hipSuccess && side_tail) e = side_tail(p, side);
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, MODE, DROP, G>), gkv, dim3(256), 0, s, p);
  keep(hipGetLastError());
  keep(hipStreamWaitEvent(s, ev[1], 0));
  if (e == hipSuccess && tail) e = tail(p, s);
  const hipError_t ej = hipEventRecord(ev[2], side);
  keep(ej);
  keep(ej == hipSuccess ? hipStreamWaitEvent(s, ev[2], 0) : ej);
  for (hipEvent_t x : ev) (void)hipEventDestroy(x);
  return e;
}

template <typename E, int D, typename G>
hipError_t launch_modes(const BwdParams& p, hipStream_t s, BwdTail tail, BwdTail side_tail) {
  const bool drop = p.keep != nullptr;
  switch (bmode_of(p)) {
    case B_NONE: return drop ? launch_main<E, D, B_NONE, true, G>(p, s, tail, side_tail) : launch_main<E, D, B_NONE, false, G>(p, s, tail, side_tail);
    case B_INDEX: return drop ? launch_main<E, D, B_INDEX, true, G>(p, s, tail, side_tail) : launch_main<E, D, B_INDEX, false, G>(p, s, tail, side_tail);
    case B_RELPOS:
      if (p.grid_h <= 32 && p.grid_w <= 32) {
        return drop ? launch_main<E, D, B_RELPOS, true, G, true>(p, s, tail, side_tail) : launch_main<E, D, B_RELPOS, false, G, true>(p, s, tail, side_tail);
      } else {
        return drop ? launch_main<E, D, B_RELPOS, true, G>(p, s, tail, side_tail) : launch_main<E, D, B_RELPOS, false, G>(p, s, tail, side_tail);
      }
    case B_RELPOS64:
      return drop ? launch_main<E, D, B_RELPOS64, true, G>(p, s, tail, side_tail) : launch_main<E, D, B_RELPOS64, false, G>(p, s, tail, side_tail);
    default: return drop ? launch_main<E, D, B_TENSOR, true, G>(p, s, tail, side_tail) : launch_main<E, D, B_TENSOR, false, G>(p, s, tail, side_tail);
  }
}

template <typename E, int D>
hipError_t launch_typed(const BwdParams& p, hipStream_t s, BwdTail tail, BwdTail side_tail) {
  const int64_t rows = p.B * p.Hq * p.Tq;
  const int64_t blocks = (rows * (D / 8) + 255) / 256;
  if (p.o_dtype == 0) hipLaunchKernelGGL((bwd_delta_kernel<E, float, D>), dim3((unsigned)blocks), dim3(256), 0, s, p, rows);
  else hipLaunchKernelGGL((bwd_delta_kernel<E, E, D>), dim3((unsigned)blocks), dim3(256), 0, s, p, rows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return p.grad_dtype == 0 ? launch_modes<E, D, float>(p, s, tail, side_tail) : launch_modes<E, D, E>(p, s, tail, side_tail);
}

template <typename E>
hipError_t launch_e(const BwdParams& p, hipStream_t s, BwdTail tail, BwdTail side_tail) {
  if (p.D == 32) return launch_typed<E, 32>(p, s, tail, side_tail);
  if (p.D == 64) return launch_typed<E, 64>(p, s, tail, side_tail);
  return launch_typed<E, 128>(p, s, tail, side_tail);
}

}  // namespace

bool bwd_supports(const BwdParams& p) {
  if (p.dtype != 1 && p.dtype != 2) return false;
  if (p.D != 32 && p.D != 64 && p.D != 128) return false;
  if (bmode_of(p) < 0) return false;
  if (p.bias == BIAS_RELPOS && (p.grid_w < 4 || p.grid_h < 1 || p.grid_h + p.grid_w > kMaxGT ||
                                p.B * p.Hq > 65535))
    return false;
  if (p.B * p.Hq * p.Tq * (p.D / 8) / 256 + 1 > INT32_MAX) return false;
  return true;
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t s, BwdTail tail, BwdTail side_tail) {
  return p.dtype == 2 ? launch_e<_Float16>(p, s, tail, side_tail) : launch_e<__bf16>(p, s, tail, side_tail);
}

}  // namespace sdpa
