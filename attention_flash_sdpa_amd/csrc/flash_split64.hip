// head_dim-64 flash attention for shapes with few query rows per GPU, such as
// SAM ViT-B's 64x64 global attention (12 heads x 4096 queries = 1536 blocks of
// 32 rows for 1024 SIMDs), with no mask or the decomposed rel-pos bias.
//
//   O = softmax(Q . K^T * scale + B) . V   ([Axon PR 650]
//   "Axon.Layers.scaled_dot_product_attention/4", description;
//   B = term_h[q, row(k)] + term_w[q, col(k)]: [Candle PR 3280] "feat(metal):
//   SDPA with Relative Positional Embeddings & LayerNorm Stability", Key
//   Changes; [mlx-examples issue 1451] "segment_anything: fuse attention with
//   mx.fast.scaled_dot_product_attention", body).
//
// Work split.  A workgroup of 4 waves covers 64 query rows of one head: two
// 32-row query blocks times two halves of the key range.  Each wave runs the
// online softmax over its half; at the end the two halves of a query block
// are merged through LDS by their running max and sum.  The GPU then holds
// 3 workgroups per CU (12 waves, 3 per SIMD) and a 12 x 4096 problem deals
// out evenly: 768 workgroups for 256 CUs.
//
// Per 32-key tile and wave: S^T = K . Q^T (4 MFMA 32x32x16, K from LDS, Q^T in
// registers), softmax in log2 units (one query per lane), O^T += V^T . P^T
// (4 MFMAs, V^T through the transposing LDS read).  Tiles are copied from HBM
// into LDS by buffer loads that write LDS directly (no staging registers;
// rows beyond the key range read as zero), double-buffered per half.
//
// Rel-pos (64-wide grid rows): term_w / scale for the 64 columns of a grid row
// initialises the score accumulators (two 32-key tiles per grid row, one half
// of the columns each), term_h of the row is one scalar per query.  The terms
// are either formed here from Q and the tables (MFMA, as in the general
// kernel) or read from precomputed term arrays.
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
typedef __attribute__((address_space(3))) float lds_float;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;          // lazy-rescale threshold (log2 units)
constexpr float kTauSum = 256.0f;     // a tile row sum above 2^tau flags a probability that may exceed 2^tau
constexpr int BN = 32;                // keys per tile
constexpr int ROWB = 128;             // bytes per K / V row (64 16-bit elements)
constexpr int TILEB = BN * ROWB;      // 4 KB
constexpr int TH_FLOATS = 2 * 64 * 34;   // term_h^T [2 query blocks][64 y][32 q]; the half exchange uses [2][34][64]

// LDS: four distinct objects for the K / V tiles of buffer parity 0 / 1 (one
// tile per key half each) and one for term_h^T.  A step copies into the
// parity-(t+1) objects while it reads the parity-t ones; because they are
// distinct objects the compiler knows the in-flight LDS-direct copies cannot
// alias the reads, and does not stall the reads on the copies.
__shared__ __attribute__((aligned(16))) char s64_ka[2 * TILEB];
__shared__ __attribute__((aligned(16))) char s64_kb[2 * TILEB];
__shared__ __attribute__((aligned(16))) char s64_va[2 * TILEB];
__shared__ __attribute__((aligned(16))) char s64_vb[2 * TILEB];
__shared__ __attribute__((aligned(16))) float s64_th[TH_FLOATS];

enum Mode { S_NONE = 0, S_RELPOS_FUSED = 1, S_RELPOS_TERMS = 2 };

// 16 lanes read rows r..r+15 at one 16-byte chunk index: distinct bank groups.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
// Transposing reads take 4 rows x 64 contiguous bytes: flip 64-byte halves.
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

template <typename E, int MODE, bool OUT16>
__global__ __launch_bounds__(256, 3) void flash_split64_kernel(FwdParams p) {
  typedef typename Vec16<E>::x8 e8;
  typedef typename Vec16<E>::x4 e4;
  typedef typename Vec16<E>::x2 e2;
  lds_char* const ka = (lds_char*)s64_ka;
  lds_char* const kb = (lds_char*)s64_kb;
  lds_char* const va = (lds_char*)s64_va;
  lds_char* const vb = (lds_char*)s64_vb;
  lds_float* const ths = (lds_float*)s64_th;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform (scalar) index
  const int g = lane >> 5, ql = lane & 31;
  const int qb = wave & 1, hf = wave >> 1;

  // XCD-aware renumbering: each of the 8 XCDs gets a contiguous range of
  // (batch, head, query tile), so its heads' K/V stay in its own L2.
  const int64_t nblk = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int64_t lin = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t per = nblk / 8, rem = nblk % 8, xcd = lin % 8;
  const int64_t lid = xcd * per + min(xcd, rem) + lin / 8;
  const int64_t tile = lid % gridDim.x, h = (lid / gridDim.x) % gridDim.y, b = lid / ((int64_t)gridDim.x * gridDim.y);
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t wq0 = tile * 64 + 32 * qb;
  const int64_t qrow = wq0 + ql;
  const bool qvalid = qrow < p.Tq;
  const int64_t qsafe = qvalid ? qrow : 0;

  const E* qp = (const E*)p.q + b * p.q_sb + h * p.q_sh;
  e8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) qf[c] = qvalid ? *(const e8*)(qp + qrow * p.q_st + c * 16 + 8 * g) : (e8){};

  const float c2 = p.scale * kLog2e;
  // ---- rel-pos: accumulator initialisation (term_w / scale) and term_h access
  f32x16 cinit[2];
  cinit[0] = (f32x16){};
  cinit[1] = (f32x16){};
  const float* thp = nullptr;
  const lds_float* th_lds = ths + qb * (64 * 32) + ql;
  if (MODE == S_RELPOS_TERMS) {
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
  }
  if (MODE == S_RELPOS_FUSED) {
    // TH^T[y, q] = rel_pos_h[r + gh - 1 - y] . q and AW^T[m', q] = rel_pos_w[c0 + m'] . q
    // on the matrix cores; term_w[q, x] is the skewed diagonal m' = col(q) - c0 + 63 - x.
    // Both query blocks of the workgroup lie in grid row r, so the workgroup
    // first copies the rel_pos_h rows r .. r + 63 and all of rel_pos_w into LDS
    // (once per workgroup instead of once per wave), and only the waves of key
    // half 0 form the products (those of half 1 read the results).
    const int gh = p.grid_h;
    const int64_t r = wq0 / 64;
    const int c0 = (int)(wq0 % 64);
    {
      // 64 + 128 rows x 128 B = 24 KB into the tile objects (rel_pos_h rows in
      // ka, rel_pos_w rows 0..63 in kb and 64..127 in va), K-tile swizzle;
      // rows past each table read as zero (record count = table size).
      const __amdgpu_buffer_rsrc_t rhs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const E*)p.rel_h + r * 64), 0, (int)max((int64_t)0, (2 * gh - 1 - r) * 128), 0x00020000);
      const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)p.rel_w, 0, 127 * 128, 0x00020000);
#pragma unroll
      for (int j = 0; j < 6; ++j) {                 // 6 x 256 lanes x 16 B = 24 KB
        const int L = 256 * (j & 1) + tid;         // 16-byte chunk within the object (rows 0..63)
        const int row = L >> 3, pos = L & 7;
        const int trow = (j < 2 ? 0 : (j < 4 ? 0 : 64)) + row;
        const int voff = trow * 128 + ((pos ^ kswz(row)) << 4);
        lds_char* obj = j < 2 ? ka : (j < 4 ? kb : va);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 2 ? rhs : rws,
                                                 (__attribute__((address_space(3))) void*)(obj + 4096 * (j & 1) + 1024 * wave),
                                                 16, voff, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 th[2], aw[3];
    if (hf == 0) {
      // LDS row of rel_pos_h[r + gh - 1 - y] is gh - 1 - y (zero for y >= gh)
#pragma unroll
      for (int yb = 0; yb < 2; ++yb) {
        th[yb] = (f32x16){};
        const int y = yb * 32 + ql;
        const int lr = max(gh - 1 - y, 0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const e8 a = lds_b128<e8>(ka + lr * ROWB + (((2 * c + g) ^ kswz(lr)) << 4));
          th[yb] = mfma32(y < gh ? a : (e8){}, qf[c], th[yb]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 3; ++mb) {
        aw[mb] = (f32x16){};
        const int m = c0 + mb * 32 + ql;            // table row; row 127 reads as zero
        const lds_char* rowp = (m < 64 ? kb + m * ROWB : va + (m - 64) * ROWB);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          aw[mb] = mfma32(lds_b128<e8>(rowp + (((2 * c + g) ^ kswz(m & 63)) << 4)), qf[c], aw[mb]);
      }
    }
    __syncthreads();                                 // table rows no longer needed
    // Skewed gather through the term_h object, one query block at a time
    // ([32 q][97] fp32 slot), then term_h^T itself.
    const float inv_scale = 1.0f / p.scale;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (qb == pass && hf == 0) {
#pragma unroll
        for (int mb = 0; mb < 3; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) ths[ql * 97 + mb * 32 + 8 * (i / 4) + 4 * g + (i % 4)] = aw[mb][i];
      }
      __syncthreads();
      if (qb == pass) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int x = kk * 32 + 8 * (i / 4) + 4 * g + (i % 4);
            cinit[kk][i] = ths[ql * 97 + ql + 63 - x] * inv_scale;
          }
      }
      __syncthreads();
    }
    if (hf == 0) {
      lds_float* thw = ths + qb * (64 * 32);
#pragma unroll
      for (int yb = 0; yb < 2; ++yb)
#pragma unroll
        for (int i = 0; i < 16; ++i) thw[(yb * 32 + 8 * (i / 4) + 4 * g + (i % 4)) * 32 + ql] = th[yb][i];
    }
    __syncthreads();
  }

  // ---- key halves and LDS-direct tile copies
  // Half 0 takes an even number of tiles so both halves start on an even tile:
  // tile parity (which half of a 64-wide grid row) is then the unrolled step.
  const int nt = (int)((p.Tkv + BN - 1) / BN);
  const int nt0 = min(nt, (((nt + 1) / 2) + 1) & ~1);
  const int tfull = (int)(p.Tkv / BN);          // tiles with no key past the end
  const int tbeg = hf ? nt0 : 0;
  const int tend = hf ? nt : nt0;
  const int niter = nt0;                        // half 0 has at least as many tiles
  const char* kvbase = (const char*)((const E*)(qb ? p.v : p.k) + b * p.k_sb + hk * p.k_sh);
  // Key rows are addressed with 32-bit byte offsets (the launcher checks that
  // the key range spans less than 2^31 bytes).
  const int rstride = (int)(p.k_st * 2);
  const int tile_bytes = BN * rstride;
  const int span = (int)(((p.Tkv - 1) * p.k_st + 64) * 2);   // bytes from the row base to the end of the last key row
  // Wave qb of half hf copies the K (qb = 0) or V (qb = 1) tile of its half:
  // 4 instructions of 64 lanes x 16 bytes; lane data lands at LDS offset 16 * lane.
  // Per-lane byte offsets inside a tile are fixed; a per-tile descriptor moves
  // the base and shrinks the record count, so rows past the key range read 0.
  // Instruction j carries the immediate offset j * 1 KB, which moves both the
  // LDS destination and the memory address, so the memory offsets drop it.
  int voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int L = 64 * j + lane, row = L >> 3, pos = L & 7;
    voff[j] = row * rstride + ((pos ^ (qb ? vswz(row) : kswz(row))) << 4) - j * 1024;
  }
  auto stage = [&](int t, auto par) {          // tile t into the parity-PAR objects
    constexpr int PAR = decltype(par)::value;
    const int tb = t * tile_bytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kvbase + (unsigned)tb), 0, max(span - tb, 0), 0x00020000);
    auto issue = [&](lds_char* obj) {
      lds_char* dst = obj + hf * TILEB;
      __attribute__((address_space(3))) void* d = (__attribute__((address_space(3))) void*)dst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[0], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[1], 0, 1024, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[2], 0, 2048, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[3], 0, 3072, 0);
    };
    if (qb == 0) issue(PAR ? kb : ka);          // one static destination object per call site
    else issue(PAR ? vb : va);
  };

  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m = -INFINITY, l = 0.0f;
  float mz = 0.0f;                              // m, or 0 while m = -inf
  const int j16 = lane & 15, dh = (lane >> 4) & 1;
  // Tile-invariant LDS byte offsets (this half's tile included) of the
  // transposing V reads and of the K reads.
  int vro[2][2];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int row0 = 16 * tc + 4 * g + (j16 >> 2);
      vro[tc][d] = hf * TILEB + row0 * ROWB + ((((4 * d + 2 * dh + ((j16 & 3) >> 1)) ^ vswz(row0)) << 4) + ((j16 & 1) << 3));
    }
  int kro[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) kro[c] = hf * TILEB + ql * ROWB + (((2 * c + g) ^ kswz(ql)) << 4);

  auto step = [&](int t, auto par, float th_pair) {
    constexpr int PAR = decltype(par)::value;     // tile parity: buffer and grid-row half
    const lds_char* ks = PAR ? kb : ka;
    const lds_char* vs = PAR ? vb : va;
    f32x16 s = (MODE == S_NONE) ? (f32x16){} : cinit[PAR];
#pragma unroll
    for (int c = 0; c < 4; ++c) s = mfma32(lds_b128<e8>(ks + kro[c]), qf[c], s);
    // V fragments now, so their LDS latency passes under the softmax.
    e8 vf[2][2];
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const s16x4 lo4 = lds_tr(vs + vro[tc][d]);
        const s16x4 hi4 = lds_tr(vs + vro[tc][d] + 8 * ROWB);
        vf[tc][d] = __builtin_bit_cast(e8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    if (t >= tfull) {
      asm volatile("" ::: "memory");     // ragged last tile: a real branch, full tiles skip it
      const int kl0 = t * BN + 4 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (kl0 + 8 * (i / 4) + (i % 4) < (int)p.Tkv) ? s[i] : -INFINITY;
    }
    const float rowb = th_pair * kLog2e;
    // Probabilities against the running reference m (log2 units).  The tile
    // max is not computed up front: a probability above 2^tau -- detected from
    // the tile's row sum, which also catches overflow and the first tile
    // (m = -inf) -- sends the wave through the exact path, which moves m to
    // the tile max, rescales O and l, and recomputes the probabilities.
    e8 pb[2];
    auto probs = [&](float off) -> float {
      float acc = 0.0f;
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        e2 pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f32x2 pp = {fexp2(fmaf(s[8 * tc + e], c2, off)), fexp2(fmaf(s[8 * tc + e + 1], c2, off))};
          pk[e / 2] = __builtin_convertvector(pp, e2);
          acc = dot2_ones(pk[e / 2], acc);
        }
        pb[tc] = __builtin_shufflevector(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                                         __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      }
      return acc;
    };
    float lt = probs(rowb - mz);
    // (m = -inf: no key seen yet; the reference must come from an actual max)
    if (__builtin_expect((__builtin_amdgcn_ballot_w64(!(lt <= kTauSum)) | __builtin_amdgcn_ballot_w64(m == -INFINITY)) != 0, 0)) {
      float smax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
      for (int i = 4; i < 16; i += 2) smax = fmaxf(smax, fmaxf(s[i], s[i + 1]));
      smax = pair_max(smax);
      const float tmax = fmaf(smax, c2, rowb);
      const bool need = tmax > m + kTau;
      const float mn = need ? tmax : m;
      const float alpha = need ? ((m == -INFINITY) ? 0.0f : fexp2(m - mn)) : 1.0f;
      m = mn;
      mz = (m == -INFINITY) ? 0.0f : m;
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o[0][i] *= alpha;
        o[1][i] *= alpha;
      }
      lt = probs(rowb - mz);
    }
    l += lt;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int d = 0; d < 2; ++d) o[d] = mfma32(vf[tc][d], pb[tc], o[d]);
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // term_h of a grid row (two tiles), read one iteration ahead
  auto th_of = [&](int t) -> float {
    if (MODE == S_RELPOS_FUSED) return th_lds[(t >> 1) * 32];
    if (MODE == S_RELPOS_TERMS) return thp[t >> 1];
    return 0.0f;
  };
  if (tbeg < tend) stage(tbeg, P0{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float th_next = (tbeg < tend) ? th_of(tbeg) : 0.0f;
  // Steady state: every tile the body touches exists in both halves.
  const int cmin = min(nt0, nt - nt0);
  int it = 0;
  for (; it + 2 < cmin; it += 2) {
    const int t = tbeg + it;
    const float th_cur = th_next;
    th_next = th_of(t + 2);
    stage(t + 1, P1{});
    step(t, P0{}, th_cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stage(t + 2, P0{});
    step(t + 1, P1{}, th_cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (; it < niter; it += 2) {
    const int t = tbeg + it;
    const float th_cur = th_next;
    if (t + 2 < tend) th_next = th_of(t + 2);
    if (t + 1 < tend) stage(t + 1, P1{});
    if (t < tend) step(t, P0{}, th_cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < niter) {
      if (t + 2 < tend) stage(t + 2, P0{});
      if (t + 1 < tend) step(t + 1, P1{}, th_cur);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- merge the two key halves of each query block through LDS
  lds_float* xch = ths + qb * (64 * 34);
  if (hf == 1) {
    xch[lane] = m;
    xch[64 + lane] = l;
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[128 + (d * 16 + i) * 64 + lane] = o[d][i];
  }
  __syncthreads();
  if (hf == 1) return;
  const float m1 = xch[lane], l1 = xch[64 + lane];
  const float mm = fmaxf(m, m1);
  const float w0 = (m == -INFINITY) ? 0.0f : fexp2(m - mm);
  const float w1 = (m1 == -INFINITY) ? 0.0f : fexp2(m1 - mm);
  const float lt = pair_sum(fmaf(l, w0, l1 * w1));
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (!qvalid) return;
  const int64_t ob = b * p.q_sb + h * p.q_sh + qrow * p.q_st;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int dd = d * 32 + 8 * i4 + 4 * g;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e;
        v[e] = fmaf(o[d][i], w0, xch[128 + (d * 16 + i) * 64 + lane] * w1) * inv;
      }
      if (OUT16) {
        e4 vb;
#pragma unroll
        for (int e = 0; e < 4; ++e) vb[e] = (E)v[e];
        *(e4*)((E*)p.o + ob + dd) = vb;
      } else {
        *(f32x4*)((float*)p.o + ob + dd) = (f32x4){v[0], v[1], v[2], v[3]};
      }
    }
  if (p.lse && g == 0) p.lse[(b * p.Hq + h) * p.Tq + qrow] = lt > 0.0f ? (mm + __log2f(lt)) * kLn2 : -INFINITY;
}

template <typename E, int MODE>
hipError_t launch_mode(const FwdParams& p, hipStream_t s) {
  dim3 grid((unsigned)((p.Tq + 63) / 64), (unsigned)p.Hq, (unsigned)p.B);
  if (p.out_dtype != 0) hipLaunchKernelGGL((flash_split64_kernel<E, MODE, true>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((flash_split64_kernel<E, MODE, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool split64_shape_ok(const FwdParams& p) {
  if ((p.dtype != 1 && p.dtype != 2) || p.D != 64 || p.num_splits != 1) return false;
  // key rows addressed with 32-bit byte offsets
  if ((p.Tkv + BN) * p.k_st * 2 > 0x7fffffffLL) return false;
  if (p.bias == BIAS_NONE) return true;
  if (p.bias == BIAS_RELPOS) {
    if (p.grid_w != 64 || p.Tkv != p.Tq) return false;
    if (p.term_h && p.term_w) return true;
    return p.grid_h >= 1 && p.grid_h <= 64 && p.rel_h && p.rel_w;
  }
  return false;
}

bool split64_supports(const FwdParams& p) {
  // worth it when the query blocks leave SIMDs idle: fewer than ~4 blocks of 32 rows per SIMD
  return split64_shape_ok(p) && p.B * p.Hq * ((p.Tq + 31) / 32) <= 4096;
}

template <typename E>
static hipError_t launch_s64_e(const FwdParams& p, hipStream_t s) {
  if (p.bias == BIAS_RELPOS) return p.term_h ? launch_mode<E, S_RELPOS_TERMS>(p, s) : launch_mode<E, S_RELPOS_FUSED>(p, s);
  return launch_mode<E, S_NONE>(p, s);
}

hipError_t launch_split64(const FwdParams& p, hipStream_t s) {
  return p.dtype == 2 ? launch_s64_e<_Float16>(p, s) : launch_s64_e<__bf16>(p, s);
}

}  // namespace sdpa
