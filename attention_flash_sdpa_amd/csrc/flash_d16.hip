// head_dim 16 attention with several heads packed into one MFMA tile, plus
// split-KV with a log-sum-exp merge.
//
// [Candle PR 3280] "feat(metal): SDPA with Relative Positional Embeddings &
// LayerNorm Stability", Key Changes: SDPA for head_dim 16 with a packed
// vector kernel that processes two heads per SIMD group.  On gfx950 a wave
// is 64 lanes and the 16-bit matrix op is 32x32x16, whose 16-deep contraction
// is exactly one head of 16 dims; this file packs FOUR heads per wave:
//
//  * Query packing (few queries, long key range -- e.g. SAM's mask decoder,
//    7 tokens attending 4096 image tokens): the 32 score columns are
//    4 heads x 8 queries.  S^T[key, (h, t)] = sum_{(h', d)} K'[key, (h', d)]
//    Q'^T[(h', d), (h, t)] with Q'^T block-sparse (nonzero only for h' = h),
//    so one 64-deep contraction (4 MFMAs) scores 32 keys for all 4 heads.
//    P.V contracts over keys shared by every head; output rows (h, d) are
//    read back only where they meet their own head's columns.  The key range
//    can be cut into chunks (split-KV) whose partial (O, m, l) are merged.
//  * Key packing (few keys -- e.g. 4096 image tokens attending 7 tokens):
//    the 32 score rows are 4 heads x 8 keys with a block-diagonal K', the
//    columns are 32 query positions shared by the 4 heads; P.V is
//    block-diagonal as well, so only the 2 diagonal 32x32 blocks are formed.
//
// Definition followed: [Axon PR 650] "Axon.Layers.scaled_dot_product_attention/4",
// description (softmax(Q . K^T * scale + mask) . V; masks; grouped-query heads).
#include "common.h"
#include "elem16.h"

namespace sdpa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float xor32_max(float v) { return fmaxf(v, __shfl_xor(v, 32)); }
__device__ __forceinline__ float xor32_sum(float v) { return v + __shfl_xor(v, 32); }

// Mask families, one kernel instance each: no mask (only the key range),
// index masks (causal / sliding), tensor masks (additive / bool).  Keeping
// them apart keeps each instance's code small; these kernels run few waves
// per CU, so a large kernel waits on instruction fetch more than on anything.
enum MaskFamily { MF_NONE = 0, MF_INDEX = 1, MF_TENSOR = 2 };

template <int MF>
__device__ __forceinline__ float bias_of(const FwdParams& p, int64_t b, int64_t h, int64_t i, int64_t j, bool ok) {
  if (!ok) return -INFINITY;
  if (MF == MF_NONE) return 0.0f;
  if (MF == MF_INDEX) return index_allowed(p.bias, i, j, p.offset, p.window) ? 0.0f : -INFINITY;
  return tensor_mask_bias(p, b, h, i, j);
}

// ------------------------------------------------------------ query packing
// grid: (splits, ceil(Tq / 8), B * ceil(Hq / 4)); one wave per block.
// Lane column n = lane % 32 holds head hh = n / 8 of the group and query t = n % 8.
template <typename E, int MF>
__global__ __launch_bounds__(64) void d16_qpack_kernel(FwdParams p, int keys_per_split) {
  typedef typename Vec16<E>::x8 e8;
  typedef typename Vec16<E>::x4 e4;
  __shared__ __attribute__((aligned(16))) E vl[4][32][16];     // V tile: [head][key][d]
  const int lane = threadIdx.x, g = lane >> 5, n = lane & 31;
  const int hh = n >> 3, t = n & 7;
  const int64_t ngrp = (p.Hq + 3) / 4;
  const int64_t b = blockIdx.z / ngrp, h0 = (blockIdx.z % ngrp) * 4;
  const int64_t q0 = (int64_t)blockIdx.y * 8;
  const int split = blockIdx.x;
  const int64_t kbeg = (int64_t)split * keys_per_split;
  const int64_t kend = min(p.Tkv, kbeg + keys_per_split);
  const int64_t grp = p.Hq / p.Hkv;
  const int64_t hcol = h0 + hh, qcol = q0 + t;
  const bool colok = hcol < p.Hq && qcol < p.Tq;

  // Q'^T operands: chunk c carries head h0 + c, nonzero only in that head's columns.
  e8 qb[4];
  {
    e8 qv = (e8){};
    if (colok) qv = *(const e8*)((const E*)p.q + b * p.q_sb + hcol * p.q_sh + qcol * p.q_st + 8 * g);
#pragma unroll
    for (int c = 0; c < 4; ++c) qb[c] = (c == hh) ? qv : (e8){};
  }
  const float c2 = p.scale * kLog2e;
  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m = -INFINITY, l = 0.0f;

  // Tile loads go out one tile ahead: K' operands straight to registers, V as
  // 16-byte pieces that pass through LDS for the transposed operand.
  //   K' row = key k0 + (lane % 32), chunk c = head h0 + c, dims 8g..8g+7.
  //   V piece e = lane + 64r: [head r][key (lane/2)%32][half lane%2].
  // Head bases are loop invariant; heads past Hq read nothing.
  const E* kh[4];
  const E* vh[4];
  bool hok[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    hok[c] = h0 + c < p.Hq;
    const int64_t hk = (hok[c] ? h0 + c : h0) / grp;
    kh[c] = (const E*)p.k + b * p.k_sb + hk * p.k_sh + 8 * g;
    vh[c] = (const E*)p.v + b * p.k_sb + hk * p.k_sh + 8 * (lane & 1);
  }
  const int vkk = (lane >> 1) & 31;
  auto load_tile = [&](int64_t k0, e8 (&ka)[4], e8 (&vv)[4]) {
    const int64_t key = k0 + n, kj = k0 + vkk;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ka[c] = (e8){};
      if (hok[c] && key < kend) ka[c] = *(const e8*)(kh[c] + key * p.k_st);
      vv[c] = (e8){};
      if (hok[c] && kj < kend) vv[c] = *(const e8*)(vh[c] + kj * p.k_st);
    }
  };
  e8 ka[4], vv[4];
  if (kbeg < kend) load_tile(kbeg, ka, vv);
  for (int64_t k0 = kbeg; k0 < kend; k0 += 32) {
    __syncthreads();                 // previous tile's V reads are done
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + 64 * r;
      *(e8*)&vl[e >> 6][(e >> 1) & 31][8 * (e & 1)] = vv[r];
    }
    f32x16 s = (f32x16){};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = mfma32(ka[c], qb[c], s);
    if (k0 + 32 < kend) load_tile(k0 + 32, ka, vv);
    // Scores -> log2 units with masks.
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t kj = k0 + 8 * (i / 4) + 4 * g + (i % 4);
      const float bb = bias_of<MF>(p, b, hcol, qcol, kj, colok && kj < kend);
      x[i] = (bb == -INFINITY) ? -INFINITY : fmaf(s[i], c2, bb * kLog2e);
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = xor32_max(tmax);
    const float mn = fmaxf(m, tmax);
    const float alpha = (mn == -INFINITY) ? 1.0f : fexp2(m - mn);
    const float mref = (mn == -INFINITY) ? 0.0f : mn;
    m = mn;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[0][i] *= alpha;
      o[1][i] *= alpha;
    }
    e8 pb[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fexp2(x[8 * kc + e] - mref);
        l += pv;
        pb[kc][e] = (E)pv;
      }
    __syncthreads();                 // V tile visible to every lane
    // V'^T operands: rows (head 2*rb + (n/16), d = n % 16); element e <-> key
    // 16*kc + 8*(e/4) + 4*g + e%4 (the order the score registers hold keys in).
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        e8 va;
        const int hv = 2 * rb + (n >> 4), d = n & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) va[e] = vl[hv][16 * kc + 8 * (e / 4) + 4 * g + (e % 4)][d];
        o[rb] = mfma32(va, pb[kc], o[rb]);
      }
  }
  // Lane (hh, t) keeps the O^T rows of its own head: block hh / 2, rows
  // 16 * (hh % 2) + d, i.e. registers 8 * (hh % 2) + 4j + e, d = 8j + 4g + e.
  const float lt = xor32_sum(l);
  if (!colok) return;
  float ov[8];
  {
    const f32x16 blk = (hh >> 1) ? o[1] : o[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = (hh & 1) ? blk[8 + i] : blk[i];
  }
  if (p.num_splits > 1) {
    // partial: unnormalised O and (m, l) of this key chunk
    const int64_t row = ((int64_t)split * p.B + b) * p.Hq * p.Tq + hcol * p.Tq + qcol;
    float* po = p.part_o + row * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) *(f32x4*)(po + 8 * j + 4 * g) = (f32x4){ov[4 * j], ov[4 * j + 1], ov[4 * j + 2], ov[4 * j + 3]};
    if (g == 0) *(float2*)(p.part_ml + row * 2) = make_float2(m, lt);
    return;
  }
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const int64_t ob = b * p.q_sb + hcol * p.q_sh + qcol * p.q_st;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (p.out_dtype != 0) {
      e4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (E)(ov[4 * j + e] * inv);
      *(e4*)((E*)p.o + ob + 8 * j + 4 * g) = v;
    } else {
      *(f32x4*)((float*)p.o + ob + 8 * j + 4 * g) =
          (f32x4){ov[4 * j] * inv, ov[4 * j + 1] * inv, ov[4 * j + 2] * inv, ov[4 * j + 3] * inv};
    }
  }
  if (p.lse && g == 0) p.lse[(b * p.Hq + hcol) * p.Tq + qcol] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

// Merge split-KV partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One wave per (b, h, query) row, lanes over chunks: each lane folds the
// chunks s = lane, lane + 64, ... in order, then the lanes meet in a fixed
// butterfly, so the result does not depend on timing.  Every load of a row
// is issued at once (one memory round trip for up to 64 chunks).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v = fmaxf(v, __shfl_xor(v, k));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) v += __shfl_xor(v, k);
  return v;
}

template <typename E>
__global__ __launch_bounds__(256) void d16_combine_kernel(FwdParams p) {
  typedef typename Vec16<E>::x8 e8;
  const int64_t rows = p.B * p.Hq * p.Tq;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;                       // whole waves leave together
  const int S = p.num_splits;
  float ml = -INFINITY, ll = 0.0f, acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = 0.0f;
  for (int sp = lane; sp < S; sp += 64) {
    const int64_t sr = (int64_t)sp * rows + r;
    const float2 mls = *(const float2*)(p.part_ml + sr * 2);
    const f32x4* po = (const f32x4*)(p.part_o + sr * 16);
    f32x4 v[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) v[q4] = po[q4];
    if (mls.x == -INFINITY) continue;
    const float mn = fmaxf(ml, mls.x);
    const float a = (ml == -INFINITY) ? 0.0f : fexp2(ml - mn), w = fexp2(mls.x - mn);
    ml = mn;
    ll = fmaf(w, mls.y, ll * a);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * q4 + e] = fmaf(w, v[q4][e], acc[4 * q4 + e] * a);
  }
  const float M = wave_max(ml);
  const float w = (ml == -INFINITY) ? 0.0f : fexp2(ml - M);
  const float L = wave_sum(w * ll);
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = wave_sum(w * acc[d]);
  if (lane != 0) return;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t b = r / (p.Hq * p.Tq), h = (r / p.Tq) % p.Hq, i = r % p.Tq;
  const int64_t ob = b * p.q_sb + h * p.q_sh + i * p.q_st;
  if (p.out_dtype != 0) {
    e8 v0, v1;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      v0[d] = (E)(acc[d] * inv);
      v1[d] = (E)(acc[d + 8] * inv);
    }
    *(e8*)((E*)p.o + ob) = v0;
    *(e8*)((E*)p.o + ob + 8) = v1;
  } else {
    f32x4* op = (f32x4*)((float*)p.o + ob);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) op[q4] = (f32x4){acc[4 * q4] * inv, acc[4 * q4 + 1] * inv, acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv};
  }
  if (p.lse) p.lse[r] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// -------------------------------------------------------------- key packing
// grid: (ceil(Tq / 32), B * ceil(Hq / 4)); one wave per block.  Lane column
// n = lane % 32 is query q0 + n for all 4 heads; score rows are (head, key slot).
template <typename E, int MF>
__global__ __launch_bounds__(64) void d16_kpack_kernel(FwdParams p) {
  typedef typename Vec16<E>::x8 e8;
  typedef typename Vec16<E>::x4 e4;
  const int lane = threadIdx.x, g = lane >> 5, n = lane & 31;
  const int64_t ngrp = (p.Hq + 3) / 4;
  const int64_t b = blockIdx.y / ngrp, h0 = (blockIdx.y % ngrp) * 4;
  const int64_t q = (int64_t)blockIdx.x * 32 + n;
  const bool qok = q < p.Tq;
  const int64_t grp = p.Hq / p.Hkv;
  // Q'^T operands: chunk c = head h0 + c (dense over the 32 query columns).
  e8 qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qb[c] = (e8){};
    if (qok && h0 + c < p.Hq)
      qb[c] = *(const e8*)((const E*)p.q + b * p.q_sb + (h0 + c) * p.q_sh + q * p.q_st + 8 * g);
  }
  const float c2 = p.scale * kLog2e;
  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m[4], l[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
  }
  // Tile loads (K' rows and the V'^T diagonal blocks) go out one tile ahead.
  //   K' rows (head r/8, key slot r%8): block diagonal over the 4 head chunks;
  //   this lane loads only chunk hr = n / 8.
  //   V'^T block rb: rows (head 2rb + n/16, d = n%16); element e <-> (head
  //   2rb + e/4, key slot 4g + e%4); zero off the head's own slots, so this
  //   lane loads elements 4 * (n/16) + 0..3.
  const int hr = n >> 3, jr = n & 7, vhalf = n >> 4;
  const bool kok = h0 + hr < p.Hq;
  const E* kbase = (const E*)p.k + b * p.k_sb + ((kok ? h0 + hr : h0) / grp) * p.k_sh + 8 * g;
  const E* vbase[2];
  bool vok[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t hc = h0 + 2 * rb + vhalf;
    vok[rb] = hc < p.Hq;
    vbase[rb] = (const E*)p.v + b * p.k_sb + ((vok[rb] ? hc : h0) / grp) * p.k_sh + (n & 15);
  }
  auto load_tile = [&](int64_t k0, e8 (&ka)[4], e8 (&va)[2]) {
    const int64_t kr = k0 + jr;
    e8 kv = (e8){};
    if (kok && kr < p.Tkv) kv = *(const e8*)(kbase + kr * p.k_st);
#pragma unroll
    for (int c = 0; c < 4; ++c) ka[c] = (c == hr) ? kv : (e8){};
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      E t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t kj = k0 + 4 * g + e;
        t[e] = (vok[rb] && kj < p.Tkv) ? vbase[rb][kj * p.k_st] : (E)0.0f;
      }
      const E z = (E)0.0f;
      va[rb] = vhalf ? (e8){z, z, z, z, t[0], t[1], t[2], t[3]} : (e8){t[0], t[1], t[2], t[3], z, z, z, z};
    }
  };
  e8 ka[4], va[2];
  load_tile(0, ka, va);
  for (int64_t k0 = 0; k0 < p.Tkv; k0 += 8) {
    f32x16 s = (f32x16){};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = mfma32(ka[c], qb[c], s);
    const e8 vc0 = va[0], vc1 = va[1];
    if (k0 + 8 < p.Tkv) load_tile(k0 + 8, ka, va);
    // Registers 4hh..4hh+3 hold head hh, key slots 4g + 0..3.
    e8 pb[2];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int64_t hc = h0 + hh;
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t kj = k0 + 4 * g + e;
        const float bb = bias_of<MF>(p, b, hc, q, kj, qok && hc < p.Hq && kj < p.Tkv);
        x[e] = (bb == -INFINITY) ? -INFINITY : fmaf(s[4 * hh + e], c2, bb * kLog2e);
        tmax = fmaxf(tmax, x[e]);
      }
      tmax = xor32_max(tmax);
      const float mn = fmaxf(m[hh], tmax);
      const float alpha = (mn == -INFINITY) ? 1.0f : fexp2(m[hh] - mn);
      const float mref = (mn == -INFINITY) ? 0.0f : mn;
      m[hh] = mn;
      l[hh] *= alpha;
      // O^T rows of head hh: block hh/2, registers 8*(hh%2) .. +7
#pragma unroll
      for (int i = 0; i < 8; ++i) o[hh >> 1][8 * (hh & 1) + i] *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = fexp2(x[e] - mref);
        l[hh] += pv;
        pb[hh >> 1][4 * (hh & 1) + e] = (E)pv;
      }
    }
    o[0] = mfma32(vc0, pb[0], o[0]);
    o[1] = mfma32(vc1, pb[1], o[1]);
  }
  if (!qok) return;
  // Block rb, register i: head 2rb + i/8, d = 8*((i%8)/4) + 4g + i%4.
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const int64_t hc = h0 + hh;
    if (hc >= p.Hq) continue;
    const float lt = xor32_sum(l[hh]);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int64_t ob = b * p.q_sb + hc * p.q_sh + q * p.q_st;
#pragma unroll
    for (int i4 = 0; i4 < 2; ++i4) {
      const int d0 = 8 * i4 + 4 * g;
      const int reg = 8 * (hh & 1) + 4 * i4;
      if (p.out_dtype != 0) {
        e4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (E)(o[hh >> 1][reg + e] * inv);
        *(e4*)((E*)p.o + ob + d0) = v;
      } else {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[hh >> 1][reg + e] * inv;
        *(f32x4*)((float*)p.o + ob + d0) = v;
      }
    }
    if (p.lse && g == 0) p.lse[(b * p.Hq + hc) * p.Tq + q] = lt > 0.0f ? (m[hh] + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

bool d16_supports(const FwdParams& p) {
  return (p.dtype == 1 || p.dtype == 2) && p.D == 16 && p.bias != BIAS_RELPOS && (p.Tq <= 8 || p.Tkv <= 64);
}

template <typename E>
static hipError_t launch_d16_e(const FwdParams& p, hipStream_t s) {
  const int64_t ngrp = (p.Hq + 3) / 4;
  const int mf = p.bias == BIAS_NONE ? MF_NONE : (p.bias == BIAS_CAUSAL || p.bias == BIAS_SLIDING) ? MF_INDEX : MF_TENSOR;
  if (p.Tq <= 8) {
    const int splits = p.num_splits > 1 ? p.num_splits : 1;
    const int64_t kps = ((p.Tkv + splits - 1) / splits + 31) / 32 * 32;
    dim3 grid((unsigned)splits, (unsigned)((p.Tq + 7) / 8), (unsigned)(p.B * ngrp));
    if (mf == MF_NONE) hipLaunchKernelGGL((d16_qpack_kernel<E, MF_NONE>), grid, dim3(64), 0, s, p, (int)kps);
    else if (mf == MF_INDEX) hipLaunchKernelGGL((d16_qpack_kernel<E, MF_INDEX>), grid, dim3(64), 0, s, p, (int)kps);
    else hipLaunchKernelGGL((d16_qpack_kernel<E, MF_TENSOR>), grid, dim3(64), 0, s, p, (int)kps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t rows = p.B * p.Hq * p.Tq;
    hipLaunchKernelGGL((d16_combine_kernel<E>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((p.Tq + 31) / 32), (unsigned)(p.B * ngrp));
  if (mf == MF_NONE) hipLaunchKernelGGL((d16_kpack_kernel<E, MF_NONE>), grid, dim3(64), 0, s, p);
  else if (mf == MF_INDEX) hipLaunchKernelGGL((d16_kpack_kernel<E, MF_INDEX>), grid, dim3(64), 0, s, p);
  else hipLaunchKernelGGL((d16_kpack_kernel<E, MF_TENSOR>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_d16(const FwdParams& p, hipStream_t s) {
  return p.dtype == 2 ? launch_d16_e<_Float16>(p, s) : launch_d16_e<__bf16>(p, s);
}

}  // namespace sdpa
