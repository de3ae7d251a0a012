// head_dim 16 attention with several heads packed into one MFMA tile, plus
// split-KV with a log-sum-exp merge.
//
// [Candle PR 3280] "feat(metal): SDPA with Relative Positional Embeddings &
// LayerNorm Stability", Key Changes: SDPA for head_dim 16 with a packed
// vector kernel that processes two heads per SIMD group.  On gfx950 a wave
// is 64 lanes and the bf16 matrix op is 32x32x16, whose 16-deep contraction
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

namespace sdpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float xor32_max(float v) { return fmaxf(v, __shfl_xor(v, 32)); }
__device__ __forceinline__ float xor32_sum(float v) { return v + __shfl_xor(v, 32); }

// Allowed test for the index masks and the key range, plus tensor-mask bias.
__device__ __forceinline__ float bias_of(const FwdParams& p, int64_t b, int64_t h, int64_t i, int64_t j, bool qok) {
  if (!qok || j >= p.Tkv || j < 0) return -INFINITY;
  if (!index_allowed(p.bias, i, j, p.offset, p.window)) return -INFINITY;
  if (p.bias == BIAS_ADDITIVE || p.bias == BIAS_BOOL) return tensor_mask_bias(p, b, h, i, j);
  return 0.0f;
}

// ------------------------------------------------------------ query packing
// grid: (splits, ceil(Tq / 8), B * ceil(Hq / 4)); one wave per block.
// Lane column n = lane % 32 holds head hh = n / 8 of the group and query t = n % 8.
__global__ __launch_bounds__(64) void d16_qpack_kernel(FwdParams p, int keys_per_split) {
  __shared__ __attribute__((aligned(16))) __bf16 vl[4][32][16];     // V tile: [head][key][d]
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
  bf16x8 qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qb[c] = (bf16x8){};
    if (c == hh && colok) qb[c] = *(const bf16x8*)((const __bf16*)p.q + b * p.q_sb + hcol * p.q_sh + qcol * p.q_st + 8 * g);
  }
  const float c2 = p.scale * kLog2e;
  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m = -INFINITY, l = 0.0f;

  for (int64_t k0 = kbeg; k0 < kend; k0 += 32) {
    // K' operands: row = key k0 + (lane % 32), chunk c = head h0 + c, dims 8g..8g+7.
    const int64_t key = k0 + n;
    bf16x8 ka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ka[c] = (bf16x8){};
      const int64_t hc = h0 + c;
      if (hc < p.Hq && key < kend)
        ka[c] = *(const bf16x8*)((const __bf16*)p.k + b * p.k_sb + (hc / grp) * p.k_sh + key * p.k_st + 8 * g);
    }
    // Stage V for the 4 heads: 4 x 32 keys x 16 dims; lane -> (head, key pair).
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = lane + 64 * r;            // 256 16-byte pieces: [head 4][key 32][half 2]
      const int hv = e >> 6, kk = (e >> 1) & 31, half = e & 1;
      const int64_t hc = h0 + hv, kj = k0 + kk;
      bf16x8 v = (bf16x8){};
      if (hc < p.Hq && kj < kend)
        v = *(const bf16x8*)((const __bf16*)p.v + b * p.k_sb + (hc / grp) * p.k_sh + kj * p.k_st + 8 * half);
      *(bf16x8*)&vl[hv][kk][8 * half] = v;
    }
    f32x16 s = (f32x16){};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qb[c], s, 0, 0, 0);
    // Scores -> log2 units with masks.
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t kj = k0 + 8 * (i / 4) + 4 * g + (i % 4);
      const float bb = (kj < kend) ? bias_of(p, b, hcol, qcol, kj, colok) : -INFINITY;
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
    bf16x8 pb[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fexp2(x[8 * kc + e] - mref);
        l += pv;
        pb[kc][e] = (__bf16)pv;
      }
    __syncthreads();
    // V'^T operands: rows (head 2*rb + (n/16), d = n % 16); element e <-> key
    // 16*kc + 8*(e/4) + 4*g + e%4 (the order the score registers hold keys in).
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 va;
        const int hv = 2 * rb + (n >> 4), d = n & 15;
#pragma unroll
        for (int e = 0; e < 8; ++e) va[e] = vl[hv][16 * kc + 8 * (e / 4) + 4 * g + (e % 4)][d];
        o[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], o[rb], 0, 0, 0);
      }
  }
  // Lane (hh, t) keeps the O^T rows of its own head: block rb = hh / 2, rows
  // 16 * (hh % 2) + d.  Registers i with 8*(i/4) + 4g + i%4 in that range.
  const float lt = xor32_sum(l);
  const int rb = hh >> 1, base = 16 * (hh & 1);
  if (!colok) return;
  if (p.num_splits > 1) {
    // partial: unnormalised O and (m, l) of this key chunk
    const int64_t row = ((int64_t)split * p.B + b) * p.Hq * p.Tq + hcol * p.Tq + qcol;
    float* po = p.part_o + row * 16;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int r0 = 8 * i4 + 4 * g;
      if (r0 >= base && r0 < base + 16) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[rb][4 * i4 + e];
        *(f32x4*)(po + r0 - base) = v;
      }
    }
    if (g == 0) {
      p.part_ml[row * 2 + 0] = m;
      p.part_ml[row * 2 + 1] = lt;
    }
    return;
  }
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const int64_t ob = b * p.q_sb + hcol * p.q_sh + qcol * p.q_st;
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int r0 = 8 * i4 + 4 * g;
    if (r0 >= base && r0 < base + 16) {
      if (p.out_dtype == 1) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[rb][4 * i4 + e] * inv);
        *(bf16x4*)((__bf16*)p.o + ob + r0 - base) = v;
      } else {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[rb][4 * i4 + e] * inv;
        *(f32x4*)((float*)p.o + ob + r0 - base) = v;
      }
    }
  }
  if (p.lse && g == 0) p.lse[(b * p.Hq + hcol) * p.Tq + qcol] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

// Merge split-KV partials in a fixed order: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per (b, h, query) row.
__global__ __launch_bounds__(256) void d16_combine_kernel(FwdParams p) {
  const int64_t rows = p.B * p.Hq * p.Tq;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int S = p.num_splits;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, p.part_ml[((int64_t)s * rows + r) * 2]);
  float acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = 0.0f;
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const int64_t sr = (int64_t)s * rows + r;
      const float ms = p.part_ml[sr * 2];
      if (ms == -INFINITY) continue;
      const float w = fexp2(ms - M);
      L = fmaf(w, p.part_ml[sr * 2 + 1], L);
      const f32x4* po = (const f32x4*)(p.part_o + sr * 16);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = po[q4];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q4 + e] = fmaf(w, v[e], acc[4 * q4 + e]);
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t b = r / (p.Hq * p.Tq), h = (r / p.Tq) % p.Hq, i = r % p.Tq;
  const int64_t ob = b * p.q_sb + h * p.q_sh + i * p.q_st;
  if (p.out_dtype == 1) {
    __bf16* op = (__bf16*)p.o + ob;
#pragma unroll
    for (int d = 0; d < 16; ++d) op[d] = (__bf16)(acc[d] * inv);
  } else {
    float* op = (float*)p.o + ob;
#pragma unroll
    for (int d = 0; d < 16; ++d) op[d] = acc[d] * inv;
  }
  if (p.lse) p.lse[r] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// -------------------------------------------------------------- key packing
// grid: (ceil(Tq / 32), B * ceil(Hq / 4)); one wave per block.  Lane column
// n = lane % 32 is query q0 + n for all 4 heads; score rows are (head, key slot).
__global__ __launch_bounds__(64) void d16_kpack_kernel(FwdParams p) {
  const int lane = threadIdx.x, g = lane >> 5, n = lane & 31;
  const int64_t ngrp = (p.Hq + 3) / 4;
  const int64_t b = blockIdx.y / ngrp, h0 = (blockIdx.y % ngrp) * 4;
  const int64_t q = (int64_t)blockIdx.x * 32 + n;
  const bool qok = q < p.Tq;
  const int64_t grp = p.Hq / p.Hkv;
  // Q'^T operands: chunk c = head h0 + c (dense over the 32 query columns).
  bf16x8 qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qb[c] = (bf16x8){};
    if (qok && h0 + c < p.Hq)
      qb[c] = *(const bf16x8*)((const __bf16*)p.q + b * p.q_sb + (h0 + c) * p.q_sh + q * p.q_st + 8 * g);
  }
  const float c2 = p.scale * kLog2e;
  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m[4], l[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
  }
  for (int64_t k0 = 0; k0 < p.Tkv; k0 += 8) {
    // K' rows (head r/8, key slot r%8): block diagonal over the 4 head chunks.
    const int hr = n >> 3, jr = n & 7;
    const int64_t kr = k0 + jr;
    bf16x8 ka[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ka[c] = (bf16x8){};
      if (c == hr && h0 + c < p.Hq && kr < p.Tkv)
        ka[c] = *(const bf16x8*)((const __bf16*)p.k + b * p.k_sb + ((h0 + c) / grp) * p.k_sh + kr * p.k_st + 8 * g);
    }
    f32x16 s = (f32x16){};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qb[c], s, 0, 0, 0);
    // Registers 4hh..4hh+3 hold head hh, key slots 4g + 0..3.
    bf16x8 pb[2];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int64_t hc = h0 + hh;
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t kj = k0 + 4 * g + e;
        const float bb = (hc < p.Hq) ? bias_of(p, b, hc, q, kj, qok) : -INFINITY;
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
        pb[hh >> 1][4 * (hh & 1) + e] = (__bf16)pv;
      }
    }
    // V'^T, diagonal block rb: rows (head 2rb + n/16, d = n%16); element e <->
    // (head 2rb + e/4, key slot 4g + e%4); zero off the head's own slots.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int hv = 2 * rb + (n >> 4), d = n & 15;
      const int64_t hc = h0 + hv;
      bf16x8 va = (bf16x8){};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t kj = k0 + 4 * g + (e % 4);
        if ((e >> 2) == (n >> 4) && hc < p.Hq && kj < p.Tkv)
          va[e] = ((const __bf16*)p.v)[b * p.k_sb + (hc / grp) * p.k_sh + kj * p.k_st + d];
      }
      o[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[rb], o[rb], 0, 0, 0);
    }
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
      if (p.out_dtype == 1) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[hh >> 1][reg + e] * inv);
        *(bf16x4*)((__bf16*)p.o + ob + d0) = v;
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
  return p.dtype == 1 && p.D == 16 && p.bias != BIAS_RELPOS && (p.Tq <= 8 || p.Tkv <= 64);
}

hipError_t launch_d16(const FwdParams& p, hipStream_t s) {
  const int64_t ngrp = (p.Hq + 3) / 4;
  if (p.Tq <= 8) {
    const int splits = p.num_splits > 1 ? p.num_splits : 1;
    const int64_t kps = ((p.Tkv + splits - 1) / splits + 31) / 32 * 32;
    dim3 grid((unsigned)splits, (unsigned)((p.Tq + 7) / 8), (unsigned)(p.B * ngrp));
    hipLaunchKernelGGL(d16_qpack_kernel, grid, dim3(64), 0, s, p, (int)kps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t rows = p.B * p.Hq * p.Tq;
    hipLaunchKernelGGL(d16_combine_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((p.Tq + 31) / 32), (unsigned)(p.B * ngrp));
  hipLaunchKernelGGL(d16_kpack_kernel, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace sdpa
