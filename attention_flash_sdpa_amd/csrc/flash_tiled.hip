// Flash attention forward for head_dim 64 / 128, bf16 or fp16 inputs, with no
// mask, a causal / sliding-window mask or a tensor mask, grouped-query K/V
// sharing, bshd or bhsd layouts: the decoder-style path (many query rows,
// long key ranges).
//
//   O = softmax(Q . K^T * scale + M) . V     ([Axon PR 650]
//   "Axon.Layers.scaled_dot_product_attention/4", description: masks
//   {causal, offset} and {sliding_window, w, offset}; grouped-query attention
//   by repeating key/value heads).
//
// Work split.  A workgroup is 4 waves of 32 query rows.  With grouped-query
// attention the 4 waves are query heads that share one KV head at the same 32
// positions: each K/V tile in LDS feeds all of them and their mask patterns
// coincide.  Workgroups are ordered so each XCD works through a contiguous
// range of (batch, KV head) groups, heaviest (latest) query blocks first.
//
// Per 32-key tile and wave: S^T = K . Q^T (D/16 MFMA 32x32x16; K from LDS,
// Q^T in registers), online softmax in log2 units with one query per lane,
// O^T += V^T . P^T (D/32 x 2 MFMAs; V^T through the transposing LDS read).
// Tiles are copied from HBM by buffer loads that write LDS directly (rows
// past the key range read as zero), double-buffered in distinct LDS objects
// so in-flight copies never stall the reads of the current tile.  Tiles
// wholly outside a wave's causal / sliding band are skipped; only tiles the
// band boundary crosses pay for per-element masking.
//
// Tensor masks (additive fp32 / bf16, boolean bytes, contiguous along keys,
// any broadcast strides over batch, head and query) travel the same way: each
// wave copies its 32 x 32 block of the mask next to the K/V tile, XOR-swizzled
// by 16-byte chunks, and reads its 16 values per tile with 4 vector LDS reads.
//
// Decomposed rel-pos bias ([mlx-examples issue 1451] "segment_anything: fuse
// attention with mx.fast.scaled_dot_product_attention", body:
// add_decomposed_rel_pos): B[i, j] = term_h[i, j / grid_w] + term_w[i, j % grid_w]
// from the fp32 term arrays that relpos_terms wrote.  Per tile each lane reads
// its query's term_w values for its 16 keys (4 groups of 4 consecutive keys:
// with grid_w a multiple of 4 a group never crosses a grid row, so one 16-byte
// load each) and one term_h value per group, issued before the tile's Q.K^T
// products so their latency overlaps them.  Any grid_w that is a multiple of 4
// (SAM's 64 x 64 global grid at head_dim 128, other image sizes' grids).
//
// Attention dropout (no mask, causal / sliding masks or rel-pos): the weights that
// multiply V are scaled by keep / (1 - rate) while lse and the row sum stay
// those of the undropped scores ([Axon PR 650] "Axon.Layers.scaled_dot_product_attention/4",
// description: `:dropout_rate` in :train mode).  Each lane reads its row's
// keep word for the 32-key tile and zeroes its packed 16-bit weights after
// they enter the row sum; the 1 / (1 - rate) factor joins the final 1 / l.
//
// The running max is optimistic: probabilities are formed against the current
// reference and only a tile whose row sum exceeds 2^8 (a probability above
// 2^8, an overflow, or no reference yet) takes the exact path that moves the
// reference to the tile max and rescales O and the row sum.
#include "common.h"
#include "elem16.h"

#include <type_traits>

namespace sdpa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;
constexpr float kTauSum = 256.0f;
constexpr int BN = 32;
#ifndef TILED_RELPOS128_OCC2
#define TILED_RELPOS128_OCC2 1
#endif


enum Mode { T_NONE = 0, T_INDEX = 1, T_ADD_F32 = 2, T_ADD_BF16 = 3, T_BOOL = 4, T_RELPOS = 5 };

// Modes whose mask is a caller's tensor, staged in LDS beside the K/V tiles.
constexpr bool is_tensor_mode(int mode) { return mode == T_ADD_F32 || mode == T_ADD_BF16 || mode == T_BOOL; }

// Mask block geometry per mode: element size, bytes per 32-key row, 16-byte
// chunks per row, copy instructions per wave, rows per 256-byte bank sweep.
template <int MODE>
struct MCfg {
  static constexpr int ES = MODE == T_ADD_F32 ? 4 : (MODE == T_ADD_BF16 ? 2 : 1);
  static constexpr int ROWB = 32 * ES;
  static constexpr int CPR = ROWB / 16;
  static constexpr int NI = 32 * CPR / 64;
  static constexpr int WB = 32 * ROWB;                 // bytes per wave block
  static __device__ __forceinline__ int swz(int r) { return (r / (256 / ROWB)) & (CPR - 1); }
};

template <int D>
struct TCfg {
  static constexpr int ROWB = 2 * D;               // bytes per K / V row
  static constexpr int TILEB = BN * ROWB;          // bytes per tile
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int RPB = 256 / ROWB;           // rows per 256-byte bank sweep
  static constexpr int QC = D / 16;                // Q.K^T MFMA chunks
  static constexpr int DB = D / 32;                // O^T row blocks
  static constexpr int NI = TILEB / 4096;          // copy instructions per wave per tile (4 waves x 1 KB each)
  static_assert(NI <= 2, "per-lane copy offsets hold two tiles pieces");
  // 16 lanes read 16 rows at one chunk index: distinct bank groups
  static __device__ __forceinline__ int kswz(int r) { return (r / RPB) & (CH - 1); }
  // transposing reads take 4 rows x 64 bytes: distinct 64-byte groups
  static __device__ __forceinline__ int vswz(int r) { return ((r / RPB) % (4 / RPB)) << 2; }
};

template <typename V>
__device__ __forceinline__ V lds_b128(const lds_char* p) { return *(const __attribute__((address_space(3))) V*)p; }
__device__ __forceinline__ s16x4 lds_tr(const lds_char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return a > b ? a : b;
}
__device__ __forceinline__ float pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Three workgroups per CU; the head_dim-128 rel-pos instances keep the next
// tile's terms in registers as well and run two (256 registers per lane).
template <int D, int MODE>
constexpr int tiled_min_blocks() { return (MODE == T_RELPOS && D == 128 && TILED_RELPOS128_OCC2) ? 2 : 3; }

template <typename E, int D, int MODE, bool OUT16, bool DROP>
__global__ __launch_bounds__(256, (tiled_min_blocks<D, MODE>())) void flash_tiled_kernel(FwdParams p, int hpw, int64_t mask_bytes, int kps) {
  typedef typename Vec16<E>::x8 e8;
  typedef typename Vec16<E>::x4 e4;
  typedef typename Vec16<E>::x2 e2;
  constexpr bool TENSOR = is_tensor_mode(MODE);
  using M = MCfg<MODE>;
  using C = TCfg<D>;
  // Double-buffered tiles, each buffer a distinct LDS object (no false
  // dependence between copies in flight and reads of the current tile).
  __shared__ __attribute__((aligned(16))) char ft_ka[C::TILEB];
  __shared__ __attribute__((aligned(16))) char ft_kb[C::TILEB];
  __shared__ __attribute__((aligned(16))) char ft_va[C::TILEB];
  __shared__ __attribute__((aligned(16))) char ft_vb[C::TILEB];
  __shared__ __attribute__((aligned(16))) char ft_ma[TENSOR ? 4 * M::WB : 16];   // mask blocks of the 4 waves
  __shared__ __attribute__((aligned(16))) char ft_mb[TENSOR ? 4 * M::WB : 16];
  lds_char* const ka = (lds_char*)ft_ka;
  lds_char* const kb = (lds_char*)ft_kb;
  lds_char* const va = (lds_char*)ft_va;
  lds_char* const vb = (lds_char*)ft_vb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ql = lane & 31;
  const int nqb = 4 / hpw;

  // (batch, head group, query tile): XCD-contiguous ranges; within a range the
  // query tiles of a head group run from the last (heaviest for causal) down.
  const int64_t nblk = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int64_t lin = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t per = nblk / 8, rem = nblk % 8, xcd = lin % 8;
  const int64_t lid = xcd * per + min(xcd, rem) + lin / 8;
  const int64_t bx = lid % gridDim.x, hgrp = (lid / gridDim.x) % gridDim.y, bz = lid / ((int64_t)gridDim.x * gridDim.y);
  // split-KV: the z index runs over (batch, key chunk); chunk `split` holds
  // keys [split * kps, (split + 1) * kps), kps a multiple of the tile
  const int nsplit = p.num_splits > 1 ? p.num_splits : 1;
  const int64_t b = bz / nsplit, split = bz % nsplit;
  const int64_t qtile = (MODE == T_INDEX) ? (int64_t)gridDim.x - 1 - bx : bx;
  const int64_t h = hgrp * hpw + (wave % hpw);
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t wg_q0 = qtile * 32 * nqb;
  const int64_t wg_q1 = min(wg_q0 + 32 * nqb, p.Tq) - 1;
  const int64_t wq0 = wg_q0 + 32 * (wave / hpw);
  const int64_t wq1 = min(wq0 + 31, p.Tq - 1);
  const int64_t qrow = wq0 + ql;
  const bool qvalid = qrow < p.Tq;

  const E* qp = (const E*)p.q + b * p.q_sb + h * p.q_sh;
  e8 qf[C::QC];
#pragma unroll
  for (int c = 0; c < C::QC; ++c) qf[c] = qvalid ? *(const e8*)(qp + qrow * p.q_st + c * 16 + 8 * g) : (e8){};
  const float c2 = p.scale * kLog2e;

  // Rel-pos: descriptors over this (batch, head)'s term rows (reads past the
  // last row return 0; keys past the grid are masked anyway), the lane's row
  // offsets, and 1 / grid_w for the row / column split of a key.
  constexpr bool RELPOS = MODE == T_RELPOS;
  const int64_t tbh = (b * p.Hq + h) * p.Tq;
  const __amdgpu_buffer_rsrc_t ths = __builtin_amdgcn_make_buffer_rsrc(
      RELPOS ? (void*)(p.term_h + tbh * p.grid_h) : nullptr, 0, RELPOS ? (int)(p.Tq * p.grid_h * 4) : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t tws = __builtin_amdgcn_make_buffer_rsrc(
      RELPOS ? (void*)(p.term_w + tbh * p.grid_w) : nullptr, 0, RELPOS ? (int)(p.Tq * p.grid_w * 4) : 0, 0x00020000);
  int thv = 0, twv = 0;
  float rcp_gw = 0.0f;
  if (RELPOS) {
    const int qs = qvalid ? (int)qrow : 0;
    thv = qs * p.grid_h * 4;
    twv = qs * p.grid_w * 4;
    rcp_gw = 1.0f / (float)p.grid_w;
  }

  // Key tiles of the workgroup.
  int64_t lo = 0, hi = p.Tkv;
  if (MODE == T_INDEX) {
    hi = min(hi, wg_q1 + p.offset + 1);
    if (p.bias == BIAS_SLIDING) lo = max((int64_t)0, wg_q0 + p.offset - p.window + 1);
  }
  if (nsplit > 1) {
    lo = max(lo, split * kps);
    hi = min(hi, (split + 1) * kps);
  }
  const int tlo = (int)(lo / BN);
  const int thi = hi > lo ? (int)((hi + BN - 1) / BN) : tlo;
  // Allowed key interval of this lane's query: lim_lo < key <= lim_hi.
  int lim_hi = (int)(p.Tkv - 1), lim_lo = -1;
  if (MODE == T_INDEX) {
    lim_hi = (int)max(min(qrow + p.offset, p.Tkv - 1), (int64_t)-2);
    if (p.bias == BIAS_SLIDING) lim_lo = (int)min(max(qrow + p.offset - p.window, (int64_t)-1), p.Tkv);
  }

  // LDS-direct copies: every wave issues C::NI of the 1 KB pieces of each tile.
  const char* kbase = (const char*)((const E*)p.k + b * p.k_sb + hk * p.k_sh);
  const char* vbase = (const char*)((const E*)p.v + b * p.k_sb + hk * p.k_sh);
  const int rstride = (int)(p.k_st * 2);
  const int64_t span = ((p.Tkv - 1) * p.k_st + D) * 2;
  int kvo[2], vvo[2];                   // C::NI <= 2 (a dependent bound here breaks the host-side lambda capture)
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int L = 64 * (wave + 4 * j) + lane, row = L / C::CH, pos = L % C::CH;
    kvo[j] = row * rstride + ((pos ^ C::kswz(row)) << 4);
    vvo[j] = row * rstride + ((pos ^ C::vswz(row)) << 4);
  }
  // Mask block of this wave: rows wq0 .. wq0 + 31, keys of the tile; the
  // descriptor's record count ends at the mask's last element (reads past it are 0).
  const char* mbase = nullptr;
  int mvo[4] = {0, 0, 0, 0};
  if (TENSOR) {
    mbase = (const char*)p.mdata + (b * p.ms[0] + h * p.ms[1] + wq0 * p.ms[2]) * M::ES;
#pragma unroll
    for (int j = 0; j < M::NI; ++j) {
      const int L = 64 * j + lane, row = L / M::CPR, pos = L % M::CPR;
      mvo[j] = row * (int)(p.ms[2] * M::ES) + ((pos ^ M::swz(row)) << 4);
    }
  }
  auto stage = [&](int t, auto par) {
    constexpr int PAR = decltype(par)::value;
    if (TENSOR) {
      const int64_t moff = (mbase - (const char*)p.mdata) + (int64_t)t * BN * M::ES;
      const int mrec = (int)max((int64_t)0, min(mask_bytes - moff, (int64_t)0x7fffffff));
      const __amdgpu_buffer_rsrc_t mrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(mbase + (int64_t)t * BN * M::ES), 0, mrec, 0x00020000);
#pragma unroll
      for (int j = 0; j < M::NI; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            mrs, (__attribute__((address_space(3))) void*)((lds_char*)(PAR ? ft_mb : ft_ma) + M::WB * wave + 1024 * j), 16,
            mvo[j], 0, 0, 0);
    }
    const int64_t tb = (int64_t)t * BN * rstride;
    const int nrec = (int)max((int64_t)0, min(span - tb, (int64_t)0x7fffffff));
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + tb), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + tb), 0, nrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)((PAR ? kb : ka) + 1024 * (wave + 4 * j)),
                                               16, kvo[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)((PAR ? vb : va) + 1024 * (wave + 4 * j)),
                                               16, vvo[j], 0, 0, 0);
  };

  const int j16 = lane & 15, dh = (lane >> 4) & 1;
  int vro[2][C::DB];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const int row0 = 16 * tc + 4 * g + (j16 >> 2);
      vro[tc][d] = row0 * C::ROWB + ((((4 * d + 2 * dh + ((j16 & 3) >> 1)) ^ C::vswz(row0)) << 4) + ((j16 & 1) << 3));
    }
  int kro[C::QC];
#pragma unroll
  for (int c = 0; c < C::QC; ++c) kro[c] = ql * C::ROWB + (((2 * c + g) ^ C::kswz(ql)) << 4);

  f32x16 o[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) o[d] = (f32x16){};
  float m = -INFINITY, l = 0.0f;
  // Attention dropout: keep bits, one 32-bit word per 32-key tile of a score
  // row, read through a descriptor over this (batch, head)'s rows with the
  // lane's row as a 32-bit offset and the tile as the scalar offset.
  const __amdgpu_buffer_rsrc_t krs_keep = __builtin_amdgcn_make_buffer_rsrc(
      DROP ? (void*)(p.keep + (b * p.Hq + h) * p.Tq * p.keep_words) : nullptr, 0,
      DROP ? (int)(p.Tq * p.keep_words * 4) : 0, 0x00020000);
  const int keep_vo = DROP ? (int)((qvalid ? qrow : 0) * p.keep_words * 4) : 0;

  // Rel-pos terms of a tile's keys for this lane: keys t * 32 + 8 i4 + 4g + e
  // lie in grid row r, columns c .. c + 3 (one 16-byte load of term_w and one
  // term_h value per group), kept in registers until the tile is computed.
  f32x4 twn[4];
  float thn[4];
  auto load_terms = [&](int t) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int key = t * BN + 8 * i4 + 4 * g;
      // key / grid_w: key <= 2^20 and grid_w <= 1024, so the float quotient's
      // error stays far below the 0.5 / grid_w margin the half key adds
      const int r = (int)(((float)key + 0.5f) * rcp_gw);
      const int c = key - r * p.grid_w;
      twn[i4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(tws, twv + 4 * c, 0, 0));
      thn[i4] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ths, thv + 4 * r, 0, 0));
    }
  };
  if (RELPOS && tlo < thi) load_terms(tlo);

  auto step = [&](int t, auto par) {
    constexpr int PAR = decltype(par)::value;
    const int64_t k0 = (int64_t)t * BN;
    if (MODE == T_INDEX) {       // nothing allowed for this wave's rows: skip
      if (k0 > wq1 + p.offset) return;
      if (p.bias == BIAS_SLIDING && k0 + BN - 1 <= wq0 + p.offset - p.window) return;
    }
    const lds_char* ks = PAR ? kb : ka;
    const lds_char* vs = PAR ? vb : va;
    // this tile's keep bits (tiles start at multiples of 32 keys)
    const uint32_t kw = DROP ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(krs_keep, keep_vo, 4 * t, 0) : 0u;
    // Rel-pos: the bias of this lane's keys (loaded during the previous tile),
    // divided by scale, initialises the accumulator that the Q.K^T products
    // add to; then the next tile's terms are requested.
    f32x16 s;
    if (RELPOS) {
      const float inv_scale = 1.0f / p.scale;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * i4 + e] = (thn[i4] + twn[i4][e]) * inv_scale;
      if (t + 1 < thi) load_terms(t + 1);
    } else {
      s = (f32x16){};
    }
#pragma unroll
    for (int c = 0; c < C::QC; ++c) s = mfma32(lds_b128<e8>(ks + kro[c]), qf[c], s);
    if (TENSOR) {
      // this lane's 16 mask values: keys 8 * i4 + 4g + e of the tile, row ql
      const lds_char* mrow = (const lds_char*)(PAR ? ft_mb : ft_ma) + M::WB * wave + ql * M::ROWB;
      const float inv_scale = 1.0f / p.scale;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int byte = (8 * i4 + 4 * g) * M::ES;
        const lds_char* a = mrow + (((byte >> 4) ^ M::swz(ql)) << 4) + (byte & 15);
        if (MODE == T_ADD_F32) {
          const f32x4 v = *(const __attribute__((address_space(3))) f32x4*)a;
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * i4 + e] = fmaf(v[e], inv_scale, s[4 * i4 + e]);
        } else if (MODE == T_ADD_BF16) {
          const Vec16<__bf16>::x4 v = *(const __attribute__((address_space(3))) Vec16<__bf16>::x4*)a;
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * i4 + e] = fmaf((float)v[e], inv_scale, s[4 * i4 + e]);
        } else {
          const unsigned v = *(const __attribute__((address_space(3))) unsigned*)a;
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * i4 + e] = ((v >> (8 * e)) & 0xffu) ? s[4 * i4 + e] : -INFINITY;
        }
      }
    }
    bool partial = k0 + BN > p.Tkv;
    if (MODE == T_INDEX) {
      if (k0 + BN - 1 > wq0 + p.offset) partial = true;
      if (p.bias == BIAS_SLIDING && k0 <= wq1 + p.offset - p.window) partial = true;
    }
    if (partial) {
      asm volatile("" ::: "memory");     // keep a real branch: full tiles skip the mask
      const int kl0 = (int)k0 + 4 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kl0 + 8 * (i / 4) + (i % 4);
        s[i] = (key <= lim_hi && key > lim_lo) ? s[i] : -INFINITY;
      }
    }
    e8 pb[2];
    auto probs = [&](float off) -> float {
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        e2 pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2 pp = {fexp2(fmaf(s[8 * tc + e], c2, off)), fexp2(fmaf(s[8 * tc + e + 1], c2, off))};
          pk[e / 2] = __builtin_convertvector(pp, e2);
          if (e & 2) acc1 = dot2_ones(pk[e / 2], acc1);
          else acc0 = dot2_ones(pk[e / 2], acc0);
          if (DROP) {     // dropped weights leave P.V (the row sum above keeps them)
            const int i0 = 8 * tc + e;                      // even: keys i0 and i0 + 1 are adjacent
            const uint32_t two = (kw >> (8 * (i0 / 4) + 4 * g + (i0 % 4))) & 3u;
            const uint32_t msk = ((two & 1u) ? 0xFFFFu : 0u) | ((two & 2u) ? 0xFFFF0000u : 0u);
            pk[e / 2] = __builtin_bit_cast(e2, __builtin_bit_cast(uint32_t, pk[e / 2]) & msk);
          }
        }
        pb[tc] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                         __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      }
      return acc0 + acc1;
    };
    float lt = probs((m == -INFINITY) ? 0.0f : -m);
    if (__builtin_expect(__any(!(lt <= kTauSum) || m == -INFINITY), 0)) {
      float smax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
      for (int i = 4; i < 16; i += 2) smax = fmaxf(smax, fmaxf(s[i], s[i + 1]));
      smax = pair_max(smax);
      const float tmax = smax * c2;
      const bool need = tmax > m + kTau;
      const float mn = need ? tmax : m;
      const float alpha = need ? ((m == -INFINITY) ? 0.0f : fexp2(m - mn)) : 1.0f;
      m = mn;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
      lt = probs((m == -INFINITY) ? 0.0f : -m);
    }
    l += lt;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int d = 0; d < C::DB; ++d) {
        const s16x4 lo4 = lds_tr(vs + vro[tc][d]);
        const s16x4 hi4 = lds_tr(vs + vro[tc][d] + 8 * C::ROWB);
        const s16x8 a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        o[d] = mfma32(__builtin_bit_cast(e8, a8), pb[tc], o[d]);
      }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (tlo < thi) stage(tlo, P0{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = tlo; t < thi; t += 2) {
    if (t + 1 < thi) stage(t + 1, P1{});
    step(t, P0{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < thi) {
      if (t + 2 < thi) stage(t + 2, P0{});
      step(t + 1, P1{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  const float lt = pair_sum(l);
  if (!qvalid) return;
  if (nsplit > 1) {
    // this chunk's unnormalised O and (running max in log2 units, row sum)
    const int64_t prow = ((split * p.B + b) * p.Hq + h) * p.Tq + qrow;
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(f32x4*)(po + d * 32 + 8 * i4 + 4 * g) =
            (f32x4){o[d][4 * i4], o[d][4 * i4 + 1], o[d][4 * i4 + 2], o[d][4 * i4 + 3]};
    if (g == 0) *(f32x2*)(p.part_ml + prow * 2) = (f32x2){m, lt};
    return;
  }
  const float inv = lt > 0.0f ? (DROP ? p.keep_scale : 1.0f) / lt : 0.0f;
  const int64_t ob = b * p.q_sb + h * p.q_sh + qrow * p.q_st;
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int dd = d * 32 + 8 * i4 + 4 * g;
      if (OUT16) {
        e4 vb4;
#pragma unroll
        for (int e = 0; e < 4; ++e) vb4[e] = (E)(o[d][4 * i4 + e] * inv);
        *(e4*)((E*)p.o + ob + dd) = vb4;
      } else {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[d][4 * i4 + e] * inv;
        *(f32x4*)((float*)p.o + ob + dd) = v;
      }
    }
  if (p.lse && g == 0) p.lse[(b * p.Hq + h) * p.Tq + qrow] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

// Merge of the key chunks: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// M = max_s m_s.  One workgroup per output row: thread t takes head dim t % D
// and the chunks s = t / D, t / D + 256 / D, ... (at most 64 chunks: every
// load of the thread, its partials and one chunk's (m, l), is issued before
// the first wait, so the merge costs one memory round trip); the 256 / D
// partial sums of a dim then add in a fixed order, so the result does not
// depend on timing.
template <typename E, int D, bool OUT16>
__global__ __launch_bounds__(256) void tiled_combine_kernel(FwdParams p) {
  constexpr int G = 256 / D;                   // chunk groups
  constexpr int NB = 64 / G;                   // chunks per thread
  __shared__ float msh[64], lsh[64];
  __shared__ float part[G][D];
  const int tid = threadIdx.x, d = tid % D, sg = tid / D;
  const int S = p.num_splits;
  const int64_t rows = p.B * p.Hq * p.Tq;
  const int64_t r = blockIdx.x;
  f32x2 ml = {-INFINITY, 0.0f};
  if (tid < S) ml = *(const f32x2*)(p.part_ml + ((int64_t)tid * rows + r) * 2);
  float v[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int s = sg + G * u;
    v[u] = s < S ? p.part_o[((int64_t)s * rows + r) * D + d] : 0.0f;
  }
  if (tid < 64) {
    msh[tid] = ml[0];
    lsh[tid] = ml[1];
  }
  __syncthreads();
  float M = -INFINITY, L = 0.0f;
  for (int s = 0; s < S; ++s) M = fmaxf(M, msh[s]);
  for (int s = 0; s < S; ++s)
    if (msh[s] != -INFINITY) L = fmaf(fexp2(msh[s] - M), lsh[s], L);
  float acc = 0.0f;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int s = sg + G * u;
    if (s < S && msh[s] != -INFINITY) acc = fmaf(fexp2(msh[s] - M), v[u], acc);
  }
  part[sg][d] = acc;
  __syncthreads();
  if (sg != 0) return;
  float tot = 0.0f;
#pragma unroll
  for (int u = 0; u < G; ++u) tot += part[u][d];
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t b = r / (p.Hq * p.Tq), h = (r / p.Tq) % p.Hq, i = r % p.Tq;
  const int64_t ob = b * p.q_sb + h * p.q_sh + i * p.q_st + d;
  if (OUT16) ((E*)p.o)[ob] = (E)(tot * inv);
  else ((float*)p.o)[ob] = tot * inv;
  if (p.lse && d == 0) p.lse[r] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

int mask_es(const FwdParams& p) { return p.bias == BIAS_BOOL ? 1 : (p.mdtype == 0 ? 4 : 2); }

template <typename E, int D, int MODE>
hipError_t launch_t(const FwdParams& p, hipStream_t s) {
  const int64_t grp = p.Hq / p.Hkv;
  const int hpw = (grp % 4 == 0) ? 4 : (grp % 2 == 0) ? 2 : 1;
  const int64_t rows = 32 * (4 / hpw);
  const int nsplit = p.num_splits > 1 ? p.num_splits : 1;
  const int kps = (int)(((p.Tkv + nsplit - 1) / nsplit + BN - 1) / BN * BN);
  dim3 grid((unsigned)((p.Tq + rows - 1) / rows), (unsigned)(p.Hq / hpw), (unsigned)(p.B * nsplit));
  // Record count of the mask descriptors: through the end of the 16-byte chunk
  // that holds the last element.  The copies move whole chunks and the
  // descriptor zeroes every dword past the record count, so a count that
  // stopped inside the last chunk would zero the last valid elements; the
  // chunk itself (16-byte aligned, like the base) lies within the allocation's
  // last page.  Bytes past the last element land on keys >= Tkv, masked anyway.
  int64_t mask_bytes = 0;
  if (is_tensor_mode(MODE))
    mask_bytes = ((p.B - 1) * p.ms[0] + (p.Hq - 1) * p.ms[1] + (p.Tq - 1) * p.ms[2] + (p.Tkv - 1) * p.ms[3] + 1) *
                 mask_es(p);
  mask_bytes = (mask_bytes + 15) & ~(int64_t)15;
  constexpr bool CAN_DROP = MODE == T_NONE || MODE == T_INDEX || MODE == T_RELPOS;
  if (CAN_DROP && p.keep) {
    if (p.out_dtype != 0) hipLaunchKernelGGL((flash_tiled_kernel<E, D, MODE, true, CAN_DROP>), grid, dim3(256), 0, s, p, hpw, mask_bytes, kps);
    else hipLaunchKernelGGL((flash_tiled_kernel<E, D, MODE, false, CAN_DROP>), grid, dim3(256), 0, s, p, hpw, mask_bytes, kps);
  } else if (p.out_dtype != 0) {
    hipLaunchKernelGGL((flash_tiled_kernel<E, D, MODE, true, false>), grid, dim3(256), 0, s, p, hpw, mask_bytes, kps);
  } else {
    hipLaunchKernelGGL((flash_tiled_kernel<E, D, MODE, false, false>), grid, dim3(256), 0, s, p, hpw, mask_bytes, kps);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const dim3 cgrid((unsigned)(p.B * p.Hq * p.Tq));
  if (p.out_dtype != 0) hipLaunchKernelGGL((tiled_combine_kernel<E, D, true>), cgrid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((tiled_combine_kernel<E, D, false>), cgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_d(const FwdParams& p, hipStream_t s) {
  switch (p.bias) {
    case BIAS_CAUSAL:
    case BIAS_SLIDING: return launch_t<E, D, T_INDEX>(p, s);
    case BIAS_ADDITIVE: return p.mdtype == 0 ? launch_t<E, D, T_ADD_F32>(p, s) : launch_t<E, D, T_ADD_BF16>(p, s);
    case BIAS_BOOL: return launch_t<E, D, T_BOOL>(p, s);
    case BIAS_RELPOS: return launch_t<E, D, T_RELPOS>(p, s);
    default: return launch_t<E, D, T_NONE>(p, s);
  }
}

}  // namespace

bool tiled_supports(const FwdParams& p) {
  if ((p.dtype != 1 && p.dtype != 2) || (p.D != 64 && p.D != 128)) return false;
  // split-KV: no mask or causal / sliding masks, no dropout, at most 64 chunks, one merge workgroup per row
  if (p.num_splits > 1 &&
      (p.keep || p.num_splits > 64 || !(p.bias == BIAS_NONE || p.bias == BIAS_CAUSAL || p.bias == BIAS_SLIDING) ||
       p.B * p.Hq * p.Tq > 0x7fffffffLL || p.B * p.num_splits > 65535))
    return false;
  // attention dropout is built for no mask, causal / sliding masks and rel-pos
  if (p.keep && p.bias != BIAS_NONE && p.bias != BIAS_CAUSAL && p.bias != BIAS_SLIDING && p.bias != BIAS_RELPOS)
    return false;
  if (p.keep && p.Tq * p.keep_words * 4 > 0x7fffffffLL) return false;   // keep rows of a head: 32-bit offsets
  if (p.bias == BIAS_RELPOS) {
    // precomputed fp32 term arrays of one grid over one (batch, head); 16-byte
    // groups of term_w need grid_w % 4 == 0 and an aligned array; each
    // (batch, head)'s rows are addressed with 32-bit byte offsets
    if (!p.term_h || !p.term_w || p.grid_h < 1 || p.grid_w < 4 || p.grid_w % 4 != 0) return false;
    if (p.grid_h > 1024 || p.grid_w > 1024) return false;          // the row split below stays exact
    if (p.Hq != p.Hkv || p.Tq != p.Tkv || p.Tq != (int64_t)p.grid_h * p.grid_w) return false;
    if (((uintptr_t)p.term_w & 15) != 0 || ((uintptr_t)p.term_h & 3) != 0) return false;
    if (p.Tq * (int64_t)(p.grid_h > p.grid_w ? p.grid_h : p.grid_w) * 4 > 0x7fffffffLL) return false;
  } else if (p.bias == BIAS_ADDITIVE || p.bias == BIAS_BOOL) {
    // mask blocks are copied by 16-byte chunks along contiguous keys; row
    // offsets of one block and every element offset stay within 32 / 64 bits
    if (p.ms[3] != 1 || !p.mdata) return false;
    if (p.bias == BIAS_ADDITIVE && p.mdtype != 0 && p.mdtype != 1) return false;
    const int64_t es = mask_es(p);
    if (p.ms[0] < 0 || p.ms[1] < 0 || p.ms[2] < 0 || 32 * p.ms[2] * es > 0x7fffffffLL) return false;
    if (((uintptr_t)p.mdata & 15) != 0 || (p.ms[2] * es) % 16 != 0 || (p.ms[1] * es) % 16 != 0 ||
        (p.ms[0] * es) % 16 != 0)
      return false;
  } else if (p.bias != BIAS_NONE && p.bias != BIAS_CAUSAL && p.bias != BIAS_SLIDING) {
    return false;
  }
  if ((int64_t)BN * p.k_st * 2 > 0x7fffffffLL) return false;     // 32-bit byte offsets within a tile
  if (p.B > 65535 || p.Hq > 65535 || (p.Tq + 31) / 32 > 0x7fffffffLL) return false;   // grid limits
  if (p.Tkv > 0x3fffffffLL) return false;                         // key indices in 32-bit lanes
  return true;
}

hipError_t launch_tiled(const FwdParams& p, hipStream_t s) {
  if (p.dtype == 2) return p.D == 64 ? launch_d<_Float16, 64>(p, s) : launch_d<_Float16, 128>(p, s);
  return p.D == 64 ? launch_d<__bf16, 64>(p, s) : launch_d<__bf16, 128>(p, s);
}

}  // namespace sdpa
