// Attention weights for `:return_attention_weights` ([Axon PR 650]
// "Axon.Layers.scaled_dot_product_attention/4", description): the weights
// that multiply V,
//   W~[b, h, i, j] = exp(scale * q_i . k_j + bias_ij - lse_i) * Z_ij
// rebuilt from the forward pass's row log-sum-exp (so the row normalisation
// is the forward pass's own), with Z the dropout factor when keep bits are
// given and 1 otherwise.  Written as fp32 [B, Hq, Tq, Tkv].  This is a debug
// output: the T_q x T_kv write bounds it, and it runs on the vector ALUs.
//
// 16-bit inputs at head_dim 32 / 64 / 128: the scores come from the matrix
// cores (32x32x16 products, fp32 accumulation).  A workgroup is 4 waves of 32
// queries over 256 keys; each wave keeps its queries' fragments in registers
// and loads each 32-key block's K fragments straight from memory (the four
// waves read the same lines).  A lane holds one key and 16 queries of the
// block, so every store instruction writes two 128-byte row segments; the
// stores bypass the caches' retention (the output is written once).
//
// Other inputs (fp32, other head dims): one workgroup per 64 x 64 block of
// one (batch, head); the Q and K blocks are staged through LDS as fp32 and
// each thread forms a 4 x 4 patch, stored as 16-byte rows.
#include "common.h"
#include "elem16.h"

namespace sdpa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename TIN, int DMAX>
__global__ __launch_bounds__(256) void attn_weights_kernel(FwdParams p, float* out) {
  constexpr int P = DMAX + 1;              // odd pitch: conflict-free column reads
  __shared__ float qs[64 * P];
  __shared__ float ks[64 * P];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.z, b = bh / p.Hq, h = bh % p.Hq;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t i0 = (int64_t)blockIdx.y * 64, j0 = (int64_t)blockIdx.x * 64;
  const int D = (int)p.D;
  const TIN* qp = (const TIN*)p.q + b * p.q_sb + h * p.q_sh;
  const TIN* kp = (const TIN*)p.k + b * p.k_sb + hk * p.k_sh;
  for (int e = tid; e < 64 * DMAX; e += 256) {
    const int r = e / DMAX, c = e % DMAX;
    qs[r * P + c] = (i0 + r < p.Tq && c < D) ? to_f32(qp[(i0 + r) * p.q_st + c]) : 0.0f;
    ks[r * P + c] = (j0 + r < p.Tkv && c < D) ? to_f32(kp[(j0 + r) * p.k_st + c]) : 0.0f;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;  // rows 4 ty .. +3, keys 4 tx .. +3
  float acc[4][4] = {};
  for (int c = 0; c < DMAX; ++c) {
    float a[4], k4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = qs[(4 * ty + u) * P + c];
      k4[u] = ks[(4 * tx + u) * P + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], k4[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + 4 * ty + u;
    if (i >= p.Tq) continue;
    const float lse = p.lse[bh * p.Tq + i];
    const uint32_t* kr = p.keep ? p.keep + (bh * p.Tq + i) * p.keep_words : nullptr;
    float w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t j = j0 + 4 * tx + v;
      float z = acc[u][v] * p.scale;
      // conditions combined without short-circuit and applied before the exponential
      // (exp(-inf) = 0), so no score takes a branch of its own
      bool ok = (j < p.Tkv) & (lse != -INFINITY);
      if (p.bias == BIAS_CAUSAL) ok = ok & (j <= i + p.offset);
      if (p.bias == BIAS_SLIDING) ok = ok & (j <= i + p.offset) & (j > i + p.offset - p.window);
      if (p.bias == BIAS_ADDITIVE || p.bias == BIAS_BOOL) {
        if (ok) z += tensor_mask_bias(p, b, h, i, j);
      }
      float wv = __expf(ok ? z - lse : -INFINITY);
      if (kr) {      // the word index is clamped to the row, so the load needs no guard
        const uint32_t word = kr[min(j, p.Tkv - 1) >> 5];
        wv = (ok & (((word >> (j & 31)) & 1u) != 0u)) ? wv * p.keep_scale : 0.0f;
      }
      w[v] = wv;
    }
    float* orow = out + (bh * p.Tq + i) * p.Tkv + j0 + 4 * tx;
    if (j0 + 4 * tx + 3 < p.Tkv && (p.Tkv & 3) == 0) {
      *(f32x4*)orow = (f32x4){w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (j0 + 4 * tx + v < p.Tkv) orow[v] = w[v];
    }
  }
}

enum WMode { W_NONE = 0, W_INDEX = 1, W_TENSOR = 2 };

template <typename E, int D, int MODE>
__global__ __launch_bounds__(256) void attn_weights_mfma_kernel(FwdParams p, float* out) {
  typedef typename Vec16<E>::x8 e8;
  constexpr int QC = D / 16;               // 16-deep chunks of head_dim
  constexpr int KB = 8;                    // 32-key blocks per workgroup
  const int lane = threadIdx.x & 63, g = lane >> 5, nl = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bh = blockIdx.z, b = bh / p.Hq, h = bh % p.Hq;
  const int64_t hk = h / (p.Hq / p.Hkv);
  const int64_t q0 = (int64_t)blockIdx.y * 128 + 32 * wave;
  if (q0 >= p.Tq) return;                  // no workgroup barrier in this kernel: idle waves leave
  const E* qp = (const E*)p.q + b * p.q_sb + h * p.q_sh;
  const E* kp = (const E*)p.k + b * p.k_sb + hk * p.k_sh;
  // A operand of S = Q . K^T: query q0 + lane % 32, head dims 16 c + 8 (lane / 32) .. + 7
  const int64_t qa = q0 + nl;
  e8 qf[QC];
#pragma unroll
  for (int c = 0; c < QC; ++c) qf[c] = qa < p.Tq ? *(const e8*)(qp + qa * p.q_st + 16 * c + 8 * g) : (e8){};
  // result rows of this lane: queries q0 + 8 (r / 4) + 4 (lane / 32) + r % 4
  float lse[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t i = q0 + 8 * (r / 4) + 4 * g + (r % 4);
    lse[r] = i < p.Tq ? p.lse[bh * p.Tq + i] : -INFINITY;
  }
  const bool sl = p.bias == BIAS_SLIDING;
  // per-wave 32 x 32 fp32 tile for the transposed write-back; rows padded to 36 floats so
  // the two lane halves (rows 4 apart) write distinct banks and 16-byte reads stay aligned
  constexpr int TP = 36;
  __shared__ __attribute__((aligned(16))) float tiles[4][32 * TP];
  float* tw = tiles[wave];
  // 16-byte stores need 16-byte aligned rows
  const bool vec_ok = (p.Tkv % 4 == 0) && (((uintptr_t)out & 15) == 0);
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t k0 = (int64_t)blockIdx.x * (32 * KB) + 32 * kb;
    if (k0 >= p.Tkv) break;
    const int64_t j = k0 + nl;               // this lane's key
    const bool jok = j < p.Tkv;
    f32x16_e sacc = (f32x16_e){};
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const e8 kf = jok ? *(const e8*)(kp + j * p.k_st + 16 * c + 8 * g) : (e8){};
      sacc = mfma32(qf[c], kf, sacc);
    }
    // Row r of this lane is query i0 + ro(r), ro(r) = 8 (r / 4) + r % 4, i0 = q0 + 4 (lane / 32).
    // In 32-bit offsets: i < Tq iff ro < nrow; causal j <= i + offset iff ro >= -dj;
    // sliding also i + offset - j < window iff ro < window - dj (dj = i0 + offset - j, clamped).
    const int64_t i0 = q0 + 4 * g;
    const int nrow = (int)min(p.Tq - i0, (int64_t)32);
    int dlo = 0, dhi = 32;
    if (MODE == W_INDEX) {
      const int64_t dj = i0 + p.offset - j;
      dlo = (int)max(min(-dj, (int64_t)33), (int64_t)-1);
      dhi = sl ? (int)max(min(p.window - dj, (int64_t)33), (int64_t)-1) : 32;
    }
    const uint32_t* krow = p.keep ? p.keep + (bh * p.Tq + i0) * p.keep_words + (k0 >> 5) : nullptr;
    // weights of this lane's 16 (query, key) pairs into the wave's tile, row 4 (lane / 32) + ro(r)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ro = 8 * (r / 4) + (r % 4);
      const bool inb = jok & (ro < nrow);
      float z = sacc[r] * p.scale;
      bool ok = inb & (lse[r] != -INFINITY);
      if (MODE == W_INDEX) ok = ok & (ro >= dlo) & (ro < dhi);
      if (MODE == W_TENSOR) {
        if (ok) z += tensor_mask_bias(p, b, h, i0 + ro, j);
      }
      float w = __expf(ok ? z - lse[r] : -INFINITY);
      if (krow && inb) {
        const uint32_t word = krow[ro * p.keep_words];
        w = ((word >> nl) & 1u) ? w * p.keep_scale : 0.0f;
      }
      tw[(ro + 4 * g) * TP + nl] = w;
    }
    // lanes exchange values through the tile: order the writes before the reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // row-major read-back: lane l takes row 8 jj + l / 8, keys 4 (l % 8) .. + 3; each store
    // instruction writes 8 rows of 128 contiguous bytes
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = 8 * jj + (lane >> 3), c4 = 4 * (lane & 7);
      const f32x4 v = *(const f32x4*)(tw + row * TP + c4);
      const int64_t i = q0 + row, j0 = k0 + c4;
      if (i >= p.Tq) continue;
      float* o = out + (bh * p.Tq + i) * p.Tkv + j0;
      if (vec_ok && j0 + 3 < p.Tkv) {
        __builtin_nontemporal_store(v, (f32x4*)o);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < p.Tkv) __builtin_nontemporal_store(v[e], o + e);
      }
    }
    // the next block's writes come after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <typename E, int D>
void launch_mfma_d(const FwdParams& p, float* w, hipStream_t s) {
  dim3 grid((unsigned)((p.Tkv + 255) / 256), (unsigned)((p.Tq + 127) / 128), (unsigned)(p.B * p.Hq));
  if (p.bias == BIAS_CAUSAL || p.bias == BIAS_SLIDING)
    hipLaunchKernelGGL((attn_weights_mfma_kernel<E, D, W_INDEX>), grid, dim3(256), 0, s, p, w);
  else if (p.bias == BIAS_ADDITIVE || p.bias == BIAS_BOOL)
    hipLaunchKernelGGL((attn_weights_mfma_kernel<E, D, W_TENSOR>), grid, dim3(256), 0, s, p, w);
  else
    hipLaunchKernelGGL((attn_weights_mfma_kernel<E, D, W_NONE>), grid, dim3(256), 0, s, p, w);
}

template <typename E>
void launch_mfma(const FwdParams& p, float* w, hipStream_t s) {
  if (p.D == 32) launch_mfma_d<E, 32>(p, w, s);
  else if (p.D == 64) launch_mfma_d<E, 64>(p, w, s);
  else launch_mfma_d<E, 128>(p, w, s);
}

// 16-byte fragment loads: 16-byte aligned bases, element strides in multiples of 8.
bool mfma_ok(const FwdParams& p) {
  if (p.dtype != 1 && p.dtype != 2) return false;
  if (p.D != 32 && p.D != 64 && p.D != 128) return false;
  if (((uintptr_t)p.q & 15) || ((uintptr_t)p.k & 15)) return false;
  for (int64_t st : {p.q_sb, p.q_sh, p.q_st, p.k_sb, p.k_sh, p.k_st})
    if (st % 8 != 0) return false;
  return (p.Tq + 127) / 128 <= 65535;
}

template <typename TIN>
hipError_t launch_t(const FwdParams& p, float* w, hipStream_t s) {
  dim3 grid((unsigned)((p.Tkv + 63) / 64), (unsigned)((p.Tq + 63) / 64), (unsigned)(p.B * p.Hq));
  if (p.D <= 32) hipLaunchKernelGGL((attn_weights_kernel<TIN, 32>), grid, dim3(256), 0, s, p, w);
  else if (p.D <= 64) hipLaunchKernelGGL((attn_weights_kernel<TIN, 64>), grid, dim3(256), 0, s, p, w);
  else hipLaunchKernelGGL((attn_weights_kernel<TIN, 128>), grid, dim3(256), 0, s, p, w);
  return hipGetLastError();
}

}  // namespace

bool attn_weights_mfma(const FwdParams& p) { return mfma_ok(p); }

hipError_t launch_attn_weights(const FwdParams& p, float* weights, hipStream_t s) {
  if (mfma_ok(p)) {
    if (p.dtype == 2) launch_mfma<_Float16>(p, weights, s);
    else launch_mfma<__bf16>(p, weights, s);
    return hipGetLastError();
  }
  if (p.dtype == 0) return launch_t<float>(p, weights, s);
  return p.dtype == 2 ? launch_t<_Float16>(p, weights, s) : launch_t<__bf16>(p, weights, s);
}

}  // namespace sdpa
