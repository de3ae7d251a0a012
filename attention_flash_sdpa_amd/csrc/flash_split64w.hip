// head_dim-64 flash attention, one 12-wave workgroup per CU: six 32-row query
// blocks (192 queries) times two halves of the key range.  This suits shapes
// whose query rows fill the GPU in whole workgroups, such as SAM ViT-B's 64x64
// global attention (12 heads x 128 query blocks = 256 workgroups of six blocks
// for 256 CUs), with no mask or the decomposed rel-pos bias.  The query blocks
// of all (batch, head) pairs are numbered in one sequence and dealt out six at
// a time, so a workgroup may hold the last blocks of one head and the first of
// the next: it then streams the K / V tiles of both heads.
//
//   O = softmax(Q . K^T * scale + B) . V   ([Axon PR 650]
//   "Axon.Layers.scaled_dot_product_attention/4", description;
//   B = term_h[q, row(k)] + term_w[q, col(k)]: [Candle PR 3280] "feat(metal):
//   SDPA with Relative Positional Embeddings & LayerNorm Stability", Key
//   Changes; [mlx-examples issue 1451] "segment_anything: fuse attention with
//   mx.fast.scaled_dot_product_attention", body).
//
// Why one wide workgroup instead of three narrow ones per CU: the three waves
// sharing a SIMD then start every tile together after the workgroup barrier,
// and the oldest-first issue order staggers them so one wave's matrix
// products run under another's softmax.  Independent narrow workgroups drift
// against each other and lose that overlap.  The K / V tiles of each key half
// are also shared by up to six waves instead of two, which cuts the copies per
// tile.
//
// Per wave and 32-key tile: S^T = K . Q^T (4 MFMA 32x32x16, K from LDS, Q^T in
// registers), softmax in log2 units (one query per lane), O^T += V^T . P^T
// (4 MFMAs, V^T through the transposing LDS read).  Tiles are copied from HBM
// into LDS by buffer loads that write LDS directly, double-buffered; at the
// end the two key halves of each query block merge through LDS by their
// running max and sum.
//
// Rel-pos (64-wide grid rows): term_w / scale for the 64 columns of a grid row
// initialises the score accumulators (two 32-key tiles per grid row, one half
// of the columns each), term_h of the row is one scalar per query.  The terms
// are either formed here from Q and the tables (MFMA) or read from
// precomputed term arrays.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;          // lazy-rescale threshold (log2 units)
constexpr float kTauSum = 256.0f;     // a tile row sum above 2^tau flags a probability that may exceed 2^tau
constexpr int NQB = 6;                // query blocks of 32 rows per workgroup
constexpr int NW = 2 * NQB;           // waves
constexpr int QROWS = 32 * NQB;       // query rows per workgroup
constexpr int BN = 32;                // keys per tile
constexpr int ROWB = 128;             // bytes per K / V row (64 16-bit elements)
constexpr int TILEB = BN * ROWB;      // 4 KB
constexpr int GSLOT = 32 * 97;        // floats of one query block's term_w gather slot
constexpr int UBYTES = 3 * GSLOT * 4;     // shared region: tables / gather slots / merge exchange (3 blocks at a time)

// LDS.  Two distinct objects for the K / V tiles of buffer parity 0 / 1, each
// [head slot][K, V][key half][tile]: a step copies into the parity-(t+1)
// object while it reads the parity-t one, and because they are distinct
// objects the compiler knows the in-flight LDS-direct copies cannot alias the
// reads.  term_h^T per query block [y][32 q] for the whole kernel; one region
// that holds in turn the rel-pos tables, the term_w gather slots and the
// merge exchange.
__shared__ __attribute__((aligned(16))) char w64_t0[8 * TILEB];
__shared__ __attribute__((aligned(16))) char w64_t1[8 * TILEB];
// byte offset of a tile in a parity object
__host__ __device__ constexpr int tile_off(int hs, int kv, int half) { return ((2 * hs + kv) * 2 + half) * TILEB; }
__shared__ __attribute__((aligned(16))) float w64_th[NQB * 64 * 32];
__shared__ __attribute__((aligned(16))) char w64_u[UBYTES];

static_assert(UBYTES >= 2 * 128 * ROWB, "tables fit the shared region");
static_assert(UBYTES >= 3 * 34 * 64 * 4, "merge exchange fits the shared region");

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
__global__ __launch_bounds__(64 * NW, 1) void flash_split64w_kernel(FwdParams p) {
  typedef typename Vec16<E>::x8 e8;
  typedef typename Vec16<E>::x4 e4;
  typedef typename Vec16<E>::x2 e2;
  lds_char* const tp0 = (lds_char*)w64_t0;
  lds_char* const tp1 = (lds_char*)w64_t1;
  lds_float* const ths = (lds_float*)w64_th;
  lds_char* const ureg = (lds_char*)w64_u;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);     // wave-uniform (scalar) index
  const int g = lane >> 5, ql = lane & 31;
  const int qb = wave % NQB, hf = wave / NQB;

  // XCD-aware renumbering: each of the 8 XCDs gets a contiguous range of
  // workgroups, so its heads' K/V stay in its own L2.
  const int64_t nwg = gridDim.x;
  const int64_t lin = blockIdx.x;
  const int64_t per = nwg / 8, rem = nwg % 8, xcd = lin % 8;
  const int64_t lid = xcd * per + min(xcd, rem) + lin / 8;
  // Query block sequence over (batch, head, block); this wave's block, and
  // the (batch, head) of the workgroup's first block (head slot 0).  A head
  // has at least 5 blocks, so six consecutive blocks span at most two heads.
  const int64_t nbh = (p.Tq + 31) / 32;
  const int64_t nball = p.B * p.Hq * nbh;
  const int64_t fb0 = lid * NQB;
  const int64_t fb = min(fb0 + qb, nball - 1);
  const int64_t bh = fb / nbh, bh0 = fb0 / nbh;
  const int hs = bh != bh0;                        // head slot of this wave's query block
  const int64_t b = bh / p.Hq, h = bh % p.Hq;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t wq0 = (fb % nbh) * 32;
  const int64_t qrow = wq0 + ql;
  const bool qvalid = fb0 + qb < nball && qrow < p.Tq;
  const int64_t qsafe = qvalid ? qrow : 0;
  // the workgroup holds a second head if its last block lies beyond the first head
  const bool two = min(fb0 + NQB - 1, nball - 1) / nbh != bh0;

  // ---- key halves and the tile-copy roles
  // Half 0 takes an even number of tiles so both halves start on an even tile:
  // tile parity (which half of a 64-wide grid row) is then the unrolled step.
  const int nt = (int)((p.Tkv + BN - 1) / BN);
  const int nt0 = min(nt, (((nt + 1) / 2) + 1) & ~1);
  const int tfull = (int)(p.Tkv / BN);          // tiles with no key past the end
  const int tbeg = hf ? nt0 : 0;
  const int tend = hf ? nt : nt0;
  const int niter = nt0;                        // half 0 has at least as many tiles
  // Copies per tile step, each a whole 4 KB K or V (dk) tile of one key half
  // (dh).  They go to the oldest waves of each SIMD (waves w, w + 4, w + 8
  // share one), which otherwise wait longest at the step's barrier: waves
  // 0..3 copy head slot 0, waves 4..7 head slot 1 in a workgroup holding two
  // heads, waves 8..11 nothing.  Key rows are addressed with 32-bit byte
  // offsets (the launcher checks that the key range spans less than 2^31
  // bytes).
  const bool cslot1 = wave >= 4;
  const bool copier = wave < 4 || (wave < 8 && two);
  const int dh = (wave >> 1) & 1, dk = wave & 1;
  const int dtbeg = dh ? nt0 : 0, dtend = dh ? nt : nt0;
  const int64_t cbh = (cslot1 && two) ? bh0 + 1 : bh0;   // (batch, head) whose tiles this wave copies
  const int64_t chk = (cbh % p.Hq) / (p.Hq / p.Hkv);
  const char* kvbase = (const char*)((const E*)(dk ? p.v : p.k) + (cbh / p.Hq) * p.k_sb + chk * p.k_sh);
  const int rstride = (int)(p.k_st * 2);
  const int tile_bytes = BN * rstride;
  const int span = (int)(((p.Tkv - 1) * p.k_st + 64) * 2);   // bytes from the row base to the end of the last key row
  // Instructions of 64 lanes x 16 bytes; lane data lands at LDS offset
  // 16 * lane.  Instruction j carries the immediate offset j * 1 KB, which
  // moves both the LDS destination and the memory address, so the memory
  // offsets drop it.  A per-tile descriptor moves the base and shrinks the
  // record count, so rows past the key range read 0.
  int voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int L = 64 * j + lane, row = L >> 3, pos = L & 7;
    voff[j] = row * rstride + ((pos ^ (dk ? vswz(row) : kswz(row))) << 4) - j * 1024;
  }
  const int dst = tile_off(cslot1 ? 1 : 0, dk, dh);   // byte offset in a parity object
  // Copy role, fixed per wave: 0 none, 1 a whole tile.  The main loop is
  // instantiated per role, so no step branches on it.
  const int role = copier ? 1 : 0;
  // Tile it of the copier's half into the parity-PAR object (GUARD: skip tiles
  // past the half's end).
  auto stage = [&](int it, auto par, auto rl, auto guard) {
    constexpr int PAR = decltype(par)::value;
    constexpr int ROLE = decltype(rl)::value;
    if (ROLE == 0) return;
    const int t = dtbeg + it;
    if (decltype(guard)::value && t >= dtend) return;
    const int tb = t * tile_bytes;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kvbase + (unsigned)tb), 0, max(span - tb, 0), 0x00020000);
    lds_void* d = (lds_void*)((PAR ? tp1 : tp0) + dst);     // one static destination object per call site
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[0], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[1], 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[2], 0, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[3], 0, 3072, 0);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using R1 = std::integral_constant<int, 1>;
  using G1 = std::true_type;
  // the first tiles travel during the set-up below
  if (role == 1) stage(0, P0{}, R1{}, G1{});

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
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 t = *(const f32x4*)(twp + kk * 32 + 8 * i4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) cinit[kk][4 * i4 + e] = t[e] * inv_scale;
      }
    thp = p.term_h + ((b * p.Hq + h) * p.Tq + qsafe) * p.grid_h;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                             // the first tiles are in LDS
  }
  if (MODE == S_NONE) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (MODE == S_RELPOS_FUSED) {
    // TH^T[y, q] = rel_pos_h[R + gh - 1 - y] . q and AW^T[m', q] = rel_pos_w[c0 + m'] . q
    // on the matrix cores (R, c0: grid row and first column of the block);
    // term_w[q, x] is the skewed diagonal m' = col(q) - c0 + 63 - x.  The
    // workgroup copies both tables whole (2 gh - 1 <= 127 and 127 rows; row
    // 127 and rows past a shorter rel_pos_h read as zero) into the shared
    // region once; the waves of key half 1 form the term_h products, those of
    // half 0 the term_w products.
    const int gh = p.grid_h;
    const int R = (int)(wq0 / 64);
    const int c0 = (int)(wq0 % 64);
    {
      const __amdgpu_buffer_rsrc_t rhs =
          __builtin_amdgcn_make_buffer_rsrc((void*)p.rel_h, 0, (2 * gh - 1) * 128, 0x00020000);
      const __amdgpu_buffer_rsrc_t rws = __builtin_amdgcn_make_buffer_rsrc((void*)p.rel_w, 0, 127 * 128, 0x00020000);
      // 2 x 128 rows x 8 chunks = 2048 chunks of 16 bytes: chunk L = 768 j + tid
      // (waves 8..11 skip j = 2); rel_pos_h rows in [0, 16 KB), rel_pos_w in [16, 32 KB).
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (j == 2 && wave >= 8) break;
        const int L0 = 768 * j + 64 * wave;      // first chunk of this wave's instruction (wave-uniform)
        const bool wpart = L0 >= 1024;
        const int L = L0 + lane - (wpart ? 1024 : 0), row = L >> 3, pos = L & 7;
        const int voffc = row * 128 + ((pos ^ kswz(row)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wpart ? rws : rhs, (lds_void*)(ureg + 16 * L0), 16, voffc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                             // tables and the first tiles are in LDS
    const lds_char* tabh = ureg;
    const lds_char* tabw = ureg + 128 * ROWB;
    f32x16 th[2], aw[3];
    if (hf == 1) {
#pragma unroll
      for (int yb = 0; yb < 2; ++yb) {
        th[yb] = (f32x16){};
        const int y = yb * 32 + ql;
        const int lr = max(R + gh - 1 - y, 0);   // zero operand for y >= gh
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const e8 a = lds_b128<e8>(tabh + lr * ROWB + (((2 * c + g) ^ kswz(lr)) << 4));
          th[yb] = mfma32(y < gh ? a : (e8){}, qf[c], th[yb]);
        }
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 3; ++mb) {
        aw[mb] = (f32x16){};
        const int mr = c0 + mb * 32 + ql;           // table row; row 127 reads as zero
#pragma unroll
        for (int c = 0; c < 4; ++c)
          aw[mb] = mfma32(lds_b128<e8>(tabw + mr * ROWB + (((2 * c + g) ^ kswz(mr)) << 4)), qf[c], aw[mb]);
      }
    }
    __syncthreads();                             // tables no longer needed
    if (hf == 1) {
      lds_float* thw = ths + qb * (64 * 32);
#pragma unroll
      for (int yb = 0; yb < 2; ++yb)
#pragma unroll
        for (int i = 0; i < 16; ++i) thw[(yb * 32 + 8 * (i / 4) + 4 * g + (i % 4)) * 32 + ql] = th[yb][i];
    }
    // Skewed gather through [32 q][97] slots, three query blocks per pass.
    const float inv_scale = 1.0f / p.scale;
    lds_float* slot = (lds_float*)ureg + (qb % 3) * GSLOT;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const bool mine = qb / 3 == pass;
      if (mine && hf == 0) {
#pragma unroll
        for (int mb = 0; mb < 3; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) slot[ql * 97 + mb * 32 + 8 * (i / 4) + 4 * g + (i % 4)] = aw[mb][i];
      }
      __syncthreads();
      if (mine) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int x = kk * 32 + 8 * (i / 4) + 4 * g + (i % 4);
            cinit[kk][i] = slot[ql * 97 + ql + 63 - x] * inv_scale;
          }
      }
      __syncthreads();
    }
  }

  f32x16 o[2] = {(f32x16){}, (f32x16){}};
  float m = -INFINITY, l = 0.0f;
  float mz = 0.0f;                              // m, or 0 while m = -inf
  const int j16 = lane & 15, dhl = (lane >> 4) & 1;
  // Tile-invariant LDS byte offsets (this half's tile included) of the
  // transposing V reads and of the K reads.
  int vro[2][2];
#pragma unroll
  for (int tc = 0; tc < 2; ++tc)
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int row0 = 16 * tc + 4 * g + (j16 >> 2);
      vro[tc][d] = tile_off(hs, 0, hf) + row0 * ROWB + ((((4 * d + 2 * dhl + ((j16 & 3) >> 1)) ^ vswz(row0)) << 4) + ((j16 & 1) << 3));
    }
  int kro[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) kro[c] = tile_off(hs, 0, hf) + ql * ROWB + (((2 * c + g) ^ kswz(ql)) << 4);

  auto step = [&](int t, auto par, float th_pair, auto ragged) {
    constexpr int PAR = decltype(par)::value;     // tile parity: buffer and grid-row half
    const lds_char* ks = PAR ? tp1 : tp0;
    const lds_char* vs = (PAR ? tp1 : tp0) + tile_off(0, 1, 0);
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
    if (decltype(ragged)::value && t >= tfull) {
      asm volatile("" ::: "memory");     // ragged last tile: a real branch, full tiles skip it
      const int kl0 = t * BN + 4 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (kl0 + 8 * (i / 4) + (i % 4) < (int)p.Tkv) ? s[i] : -INFINITY;
    }
    // The softmax runs at raised wave priority: it is the part of a step the
    // other waves of the SIMD cannot hide (their matrix ops run under it), so
    // its instructions go first when several waves are ready to issue.
    __builtin_amdgcn_s_setprio(1);
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
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int d = 0; d < 2; ++d) o[d] = mfma32(vf[tc][d], pb[tc], o[d]);
  };

  // term_h of a grid row (two tiles), read one iteration ahead
  auto th_of = [&](int t) -> float {
    if (MODE == S_RELPOS_FUSED) return th_lds[(t >> 1) * 32];
    if (MODE == S_RELPOS_TERMS) return thp[t >> 1];
    return 0.0f;
  };
  float th_next = (tbeg < tend) ? th_of(tbeg) : 0.0f;
  using G0 = std::false_type;
  auto main_loop = [&](auto rl) {
    // Steady state: every tile the body touches exists in both halves and is
    // full (only the last tile of the key range can be ragged).
    const int cmin = min(nt0, nt - nt0);
    int it = 0;
    for (; it + 2 < cmin; it += 2) {
      const int t = tbeg + it;
      const float th_cur = th_next;
      th_next = th_of(t + 2);
      stage(it + 1, P1{}, rl, G0{});
      step(t, P0{}, th_cur, G0{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      stage(it + 2, P0{}, rl, G0{});
      step(t + 1, P1{}, th_cur, G0{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    for (; it < niter; it += 2) {
      const int t = tbeg + it;
      const float th_cur = th_next;
      if (t + 2 < tend) th_next = th_of(t + 2);
      stage(it + 1, P1{}, rl, G1{});
      if (t < tend) step(t, P0{}, th_cur, G1{});
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (it + 1 < niter) {
        stage(it + 2, P0{}, rl, G1{});
        if (t + 1 < tend) step(t + 1, P1{}, th_cur, G1{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  };
  if (role == 1) main_loop(R1{});
  else main_loop(std::integral_constant<int, 0>{});

  // ---- merge the two key halves of each query block through LDS, three
  // query blocks per pass (the exchange reuses the shared region; with an
  // empty key range no loop barrier has separated it from the gather reads)
  if (niter == 0) __syncthreads();
  lds_float* xch = (lds_float*)ureg + (qb % 3) * (64 * 34);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const bool mine = qb / 3 == pass;
    if (mine && hf == 1) {
      xch[lane] = m;
      xch[64 + lane] = l;
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[128 + (d * 16 + i) * 64 + lane] = o[d][i];
    }
    __syncthreads();
    if (mine && hf == 0) {
      const float m1 = xch[lane], l1 = xch[64 + lane];
      const float mm = fmaxf(m, m1);
      const float w0 = (m == -INFINITY) ? 0.0f : fexp2(m - mm);
      const float w1 = (m1 == -INFINITY) ? 0.0f : fexp2(m1 - mm);
      const float lt = pair_sum(fmaf(l, w0, l1 * w1));
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      if (qvalid) {
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
              e4 vb4;
#pragma unroll
              for (int e = 0; e < 4; ++e) vb4[e] = (E)v[e];
              *(e4*)((E*)p.o + ob + dd) = vb4;
            } else {
              *(f32x4*)((float*)p.o + ob + dd) = (f32x4){v[0], v[1], v[2], v[3]};
            }
          }
        if (p.lse && g == 0) p.lse[(b * p.Hq + h) * p.Tq + qrow] = lt > 0.0f ? (mm + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
    if (pass == 0) __syncthreads();              // pass 1 overwrites the exchange
  }
}

template <typename E, int MODE>
hipError_t launch_mode(const FwdParams& p, hipStream_t s) {
  const int64_t nball = p.B * p.Hq * ((p.Tq + 31) / 32);
  dim3 grid((unsigned)((nball + NQB - 1) / NQB));
  if (p.out_dtype != 0) hipLaunchKernelGGL((flash_split64w_kernel<E, MODE, true>), grid, dim3(64 * NW), 0, s, p);
  else hipLaunchKernelGGL((flash_split64w_kernel<E, MODE, false>), grid, dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_w_e(const FwdParams& p, hipStream_t s) {
  if (p.bias == BIAS_RELPOS) return p.term_h ? launch_mode<E, S_RELPOS_TERMS>(p, s) : launch_mode<E, S_RELPOS_FUSED>(p, s);
  return launch_mode<E, S_NONE>(p, s);
}

}  // namespace

// Shapes of the split64 kernels (any number of query blocks: the workgroups
// are dealt out in rounds) whose heads have at least 5 query blocks (so a
// workgroup spans at most two heads) and whose workgroup count fits a 1-D
// grid; with need_fill, also only where the workgroups fill the CUs in nearly
// whole rounds (at least one full round, the rounds on average 3/4 busy).
bool split64w_supports(const FwdParams& p, bool need_fill) {
  if (!split64_shape_ok(p) || (p.Tq + 31) / 32 < 5) return false;
  const int64_t nwg = (p.B * p.Hq * ((p.Tq + 31) / 32) + NQB - 1) / NQB;
  if (nwg > 0x7fffffff) return false;
  if (!need_fill) return true;
  const int64_t cus = 256;
  if (nwg < cus) return false;
  const int64_t rounds = (nwg + cus - 1) / cus;
  return nwg * 4 >= rounds * cus * 3;
}

hipError_t launch_split64w(const FwdParams& p, hipStream_t s) {
  return p.dtype == 2 ? launch_w_e<_Float16>(p, s) : launch_w_e<__bf16>(p, s);
}

}  // namespace sdpa
