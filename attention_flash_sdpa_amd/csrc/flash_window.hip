// Windowed attention with the decomposed rel-pos bias, for SAM's 14 x 14
// windows (196 tokens, head_dim 64, bf16 or fp16): one workgroup per (window, head),
// the bias terms formed inside the kernel.
//
//   z_ij = scale * q_i . k_j + term_h[i, row(j)] + term_w[i, col(j)]
//   term_h[i, y] = q_i . Rh[row(i) - y + 13],  term_w[i, x] = q_i . Rw[col(i) - x + 13]
//
// ([mlx-examples issue 1451] "segment_anything: fuse attention with
// mx.fast.scaled_dot_product_attention", body: SAM's windowed blocks add
// add_decomposed_rel_pos's bias to the scores of each window; [Candle PR 3280]
// "feat(metal): SDPA with Relative Positional Embeddings & LayerNorm
// Stability", Key Changes: the rel-pos bias enters the fused SDPA kernel.)
//
// Layout of the work.  Seven waves of 32 query rows cover the window's 196
// rows; K and V of the whole window (25 KB each) are copied to LDS once by
// buffer loads that write LDS directly.  A key tile is two grid rows (28
// keys, padded to the 32 of the matrix op), so within a tile the key slot s
// fixes the grid column s % 14 and the row offset s / 14:
//   * term_w / scale depends only on (query, slot): it initialises the score
//     accumulators, identical for every tile (slots 28..31 start at -inf);
//   * term_h / scale depends on (query, tile, s / 14): it enters the matrix op
//     as one extra 16-deep chunk, K' rows one-hot in s / 14 against the query's
//     two term_h values of the tile, each split into a 16-bit high and low
//     part (so the bias keeps about twice the element's mantissa); the products Q . Rh^T stay
//     in LDS and each tile reads its two values.
// The terms come from two 32 x 32 x 64 products per wave, Q . Rh^T and
// Q . Rw^T over all 27 table rows, followed by a skewed gather through LDS.
//
// Placement.  Up to 256 (window, head) items, or more than 320, run one
// workgroup of seven waves per item.  In between (SAM's 25 windows x 12
// heads = 300), one workgroup per CU takes a whole item plus at most two query
// blocks of one of the items past the first 256, with both items' K and V in
// LDS.  Otherwise 44 CUs would run two whole items each and set the time.
// Every wave computes exactly as in the one-item launch, so the results are
// bitwise the same.
#include "common.h"
#include "elem16.h"

namespace sdpa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;
constexpr float kTauSum = 256.0f;

constexpr int G = 14;                 // grid side of a window
constexpr int T = G * G;              // tokens per window
constexpr int NTAB = 2 * G - 1;       // rel-pos table rows
constexpr int RPT = 32 / G;           // grid rows per key tile
constexpr int TK = RPT * G;           // keys per tile
constexpr int NT = G / RPT;           // key tiles
constexpr int NW = (T + 31) / 32;     // waves (32 query rows each)
constexpr int ROWB = 128;             // bytes per K / V row (64 16-bit elements)
constexpr int ROWS = (NT - 1) * TK + 32;   // LDS rows: the last tile reads 32 rows
constexpr int PIECES = ROWS * ROWB / 1024; // 1 KB copy pieces per tensor
static_assert(G % RPT == 0 && RPT <= 4, "tile = whole grid rows, at most 4");
static_assert(ROWS * ROWB % 1024 == 0, "copy pieces of 64 lanes x 16 B");

// Balanced launches: one workgroup per CU, each holding one whole (window,
// head) and up to two query blocks of one of the rest (see launch_window).
constexpr int CUS = 256;              // compute units of the GPU
constexpr int XNW = NW + 2;           // waves of a balanced workgroup
constexpr int XCHUNKS = 4;            // query-block chunks of an extra (window, head): 2, 2, 2, 1 blocks
static_assert(2 * (XCHUNKS - 1) + 1 == NW, "chunks cover the query blocks");

__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int vswz(int r) { return ((r >> 1) & 1) << 2; }
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

// XTRA = false: one workgroup of NW waves per (window, head), wave w taking
// query block w.  XTRA = true (balanced): CUS workgroups of XNW waves;
// workgroup j holds (window, head) j whole in waves 0..NW-1 and, for
// j < XCHUNKS * (B * H - CUS), chunk j % XCHUNKS of (window, head)
// CUS + j / XCHUNKS in waves NW, NW + 1 (blocks 2c, 2c + 1; the last chunk is
// block NW - 1 alone), each (window, head) in its own K / V slot.
template <typename E, bool OUT16, bool XTRA>
__global__ __launch_bounds__((XTRA ? XNW : NW) * 64, (XTRA ? 1 : 4)) void flash_window_kernel(FwdParams p) {
  typedef typename Vec16<E>::x8 e8;
  typedef typename Vec16<E>::x4 e4;
  typedef typename Vec16<E>::x2 e2;
  constexpr int WAVES = XTRA ? XNW : NW;
  constexpr int SLOTS = XTRA ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char fw_k[SLOTS * ROWS * ROWB];
  __shared__ __attribute__((aligned(16))) char fw_v[SLOTS * ROWS * ROWB];
  __shared__ __attribute__((aligned(16))) float fw_sc[WAVES * 32 * 32];    // per-wave [table row][query]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ql = lane & 31;
  // (window, head) items of the workgroup's K / V slots, and this wave's slot and query block
  const int64_t nitem = p.B * p.Hq;
  const int64_t item0 = blockIdx.x;
  const int64_t item1 = XTRA ? CUS + blockIdx.x / XCHUNKS : -1;
  const bool has1 = XTRA && item1 < nitem;
  const int chunk = XTRA ? (int)(blockIdx.x % XCHUNKS) : 0;
  const int slot = (XTRA && wave >= NW) ? 1 : 0;
  const int qb = slot ? 2 * chunk + (wave - NW) : wave;
  const bool active = slot == 0 || (has1 && qb < NW);
  const int64_t item = (slot && has1) ? item1 : item0;   // an unused wave reads its workgroup's first item
  const int64_t b = item / p.Hq, h = item % p.Hq;
  lds_char* const ks = (lds_char*)fw_k + slot * (ROWS * ROWB);
  lds_char* const vs = (lds_char*)fw_v + slot * (ROWS * ROWB);

  // ---- K and V of the window(s) into LDS (rows past the window read as zero)
  {
    const int rstride = (int)(p.k_st * 2);
    const int nrec = (int)(((int64_t)(T - 1) * p.k_st + 64) * 2);
    // element offsets of the slots' (batch, head) rows
    const int64_t off0 = (item0 / p.Hq) * p.k_sb + (item0 % p.Hq) * p.k_sh;
    const int64_t off1 = has1 ? (item1 / p.Hq) * p.k_sb + (item1 % p.Hq) * p.k_sh : off0;
    for (int pc = wave; pc < PIECES * (has1 ? 2 : 1); pc += WAVES) {
      const int sl = pc >= PIECES ? 1 : 0, pp = pc - sl * PIECES;
      const int64_t off = sl ? off1 : off0;
      const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)((const E*)p.k + off), 0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)((const E*)p.v + off), 0, nrec, 0x00020000);
      const int L = 64 * pp + lane, row = L >> 3, pos = L & 7;
      lds_char* const kd = (lds_char*)fw_k + sl * (ROWS * ROWB) + 1024 * pp;
      lds_char* const vd = (lds_char*)fw_v + sl * (ROWS * ROWB) + 1024 * pp;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)kd, 16,
                                               row * rstride + ((pos ^ kswz(row)) << 4), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)vd, 16,
                                               row * rstride + ((pos ^ vswz(row)) << 4), 0, 0, 0);
    }
  }

  // ---- queries of this wave, and the rel-pos table rows as matrix operands
  // (all issued together: one memory round trip; table rows past 2G-1 are zeroed)
  const int qrow = 32 * qb + ql;
  const bool qvalid = active && qrow < T;
  const int qs = qvalid ? qrow : T - 1;
  const int ih = qs / G, iw = qs % G;
  const E* qp = (const E*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)qs * p.q_st + 8 * g;
  const int trow = ql < NTAB ? ql : NTAB - 1;
  const E* rhp = (const E*)p.rel_h + trow * 64 + 8 * g;
  const E* rwp = (const E*)p.rel_w + trow * 64 + 8 * g;
  e8 qf[4], rh[4], rw[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qf[c] = *(const e8*)(qp + c * 16);
    rh[c] = *(const e8*)(rhp + c * 16);
    rw[c] = *(const e8*)(rwp + c * 16);
  }
  if (ql >= NTAB) {
#pragma unroll
    for (int c = 0; c < 4; ++c) rh[c] = rw[c] = (e8){};
  }
  const float c2 = p.scale * kLog2e;
  const float inv_scale = 1.0f / p.scale;

  // ---- rel-pos terms: A^T[r, q] = table[r] . q on the matrix cores, then the
  // skewed gathers term[q, y] = A[q, coord(q) - y + G - 1] through LDS.
  lds_float* const sc = (lds_float*)fw_sc + wave * 1024;
  auto table_product = [&](const e8 (&tab)[4]) {
    f32x16 a = (f32x16){};
#pragma unroll
    for (int c = 0; c < 4; ++c) a = mfma32(tab[c], qf[c], a);
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[(8 * (i / 4) + 4 * g + (i % 4)) * 32 + ql] = a[i];
  };
  // term_w / scale per key slot of a tile: the score accumulators' start.
  // The slot is this wave's own, so its writes and reads need only the
  // wave's own order (wave_sync), not a workgroup barrier.
  f32x16 cinit;
  table_product(rw);
  wave_sync();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int s = 8 * (i / 4) + 4 * g + (i % 4);
    const int x = s % G;
    const float t = sc[(iw - x + G - 1) * 32 + ql] * inv_scale;
    cinit[i] = s < TK ? t : -INFINITY;
  }
  wave_sync();
  // A_h stays in LDS; each tile reads its two term_h values from it.
  table_product(rh);
  // K' chunk: key slot ql (lanes g = 0) is one-hot at s / 14 and 4 + s / 14.
  e8 kaug = (e8){};
  if (g == 0 && ql < TK) {
    const int ro = ql / G;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kaug[e] = (E)(e == ro ? 1.0f : 0.0f);
      kaug[4 + e] = (E)(e == ro ? 1.0f : 0.0f);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);        // this wave's copies have landed
  __syncthreads();                      // ... and every other wave's
  if (!active) return;                  // a balanced workgroup's unused wave (no barrier follows)

  const int j16 = lane & 15, dh = (lane >> 4) & 1;
  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m = -INFINITY, l = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // Q' chunk of this tile: high parts of term_h rows RPT*t + e at e, low parts at 4 + e.
    e8 qaug = (e8){};
    if (g == 0) {
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        const float th = sc[(ih - RPT * t - e + G - 1) * 32 + ql] * inv_scale;
        const E hi = (E)th;
        qaug[e] = hi;
        qaug[4 + e] = (E)(th - (float)hi);
      }
    }
    f32x16 s = mfma32(kaug, qaug, cinit);
    const int kr = TK * t + ql;
    e8 kf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kf[c] = lds_b128<e8>(ks + kr * ROWB + (((2 * c + g) ^ kswz(kr)) << 4));
#pragma unroll
    for (int c = 0; c < 4; ++c) s = mfma32(kf[c], qf[c], s);
    // Probabilities against the running reference m; only a tile whose row
    // sum passes 2^8 (or the first tile) takes the exact path that moves m
    // to the tile max and rescales O and l.
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
      const float tmax = pair_max(smax) * c2;
      const bool need = tmax > m + kTau;
      const float mn = need ? tmax : m;
      const float alpha = need ? ((m == -INFINITY) ? 0.0f : fexp2(m - mn)) : 1.0f;
      m = mn;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
      lt = probs((m == -INFINITY) ? 0.0f : -m);
    }
    l += lt;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int row0 = TK * t + 16 * tc + 4 * g + (j16 >> 2);
        const int vo = row0 * ROWB + ((((4 * d + 2 * dh + ((j16 & 3) >> 1)) ^ vswz(row0)) << 4) + ((j16 & 1) << 3));
        const s16x4 lo4 = lds_tr(vs + vo);
        const s16x4 hi4 = lds_tr(vs + vo + 8 * ROWB);
        const s16x8 a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        o[d] = mfma32(__builtin_bit_cast(e8, a8), pb[tc], o[d]);
      }
  }

  const float lt = pair_sum(l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (!qvalid) return;
  const int64_t ob = b * p.q_sb + h * p.q_sh + (int64_t)qrow * p.q_st;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int dd = d * 32 + 8 * i4 + 4 * g;
      if (OUT16) {
        e4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (E)(o[d][4 * i4 + e] * inv);
        *(e4*)((E*)p.o + ob + dd) = v4;
      } else {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o[d][4 * i4 + e] * inv;
        *(f32x4*)((float*)p.o + ob + dd) = v4;
      }
    }
  if (p.lse && g == 0) p.lse[(b * p.Hq + h) * p.Tq + qrow] = lt > 0.0f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

}  // namespace

bool window_supports(const FwdParams& p) {
  return (p.dtype == 1 || p.dtype == 2) && p.D == 64 && p.bias == BIAS_RELPOS && !p.term_h && p.rel_h && p.rel_w &&
         p.grid_h == G && p.grid_w == G && p.Tq == T && p.Tkv == T && p.Hq == p.Hkv && p.num_splits == 1 &&
         p.B * p.Hq <= 0x7fffffffLL && (int64_t)T * p.k_st * 2 <= 0x7fffffffLL;
}

// More (window, head) items than CUs but at most CUS + CUS / XCHUNKS: the
// balanced launch (one workgroup per CU; the items past the first CUS are
// spread over the workgroups in chunks of at most two query blocks), so no CU
// runs two whole items.  Otherwise one workgroup per item.
template <typename E, bool OUT16>
void launch_window_e(const FwdParams& p, hipStream_t s) {
  const int64_t nitem = p.B * p.Hq;
  if (nitem > CUS && nitem <= CUS + CUS / XCHUNKS)
    hipLaunchKernelGGL((flash_window_kernel<E, OUT16, true>), dim3(CUS), dim3(XNW * 64), 0, s, p);
  else
    hipLaunchKernelGGL((flash_window_kernel<E, OUT16, false>), dim3((unsigned)nitem), dim3(NW * 64), 0, s, p);
}

hipError_t launch_window(const FwdParams& p, hipStream_t s) {
  if (p.dtype == 2) {
    if (p.out_dtype != 0) launch_window_e<_Float16, true>(p, s);
    else launch_window_e<_Float16, false>(p, s);
  } else {
    if (p.out_dtype != 0) launch_window_e<__bf16, true>(p, s);
    else launch_window_e<__bf16, false>(p, s);
  }
  return hipGetLastError();
}

}  // namespace sdpa
