// Attention-dropout keep bits from a counter-based generator.
//
// [Axon PR 650] "Axon.Layers.scaled_dot_product_attention/4", description:
// `:dropout_rate` drops attention probabilities in :train mode, and the graph
// layer threads a PRNG key from step to step.  Here the key is a 64-bit seed
// and the step is a 32-bit counter word, fed to Philox4x32-10 (Salmon,
// Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): score element (b, h, i, j) takes the 16-bit half j % 8 of the
// block Philox(counter = (j / 8, i, b * Hq + h, step), key = seed), low half
// of word (j % 8) / 2 first, and is kept iff that half >= thresh.
//
// Output: one 32-bit word per 32 keys of a score row, [B, Hq, Tq, ceil(Tkv / 32)],
// bit j % 32 of word j / 32; bits past Tkv are zero.  Every thread writes one
// word (four Philox blocks), so the stores are coalesced along the row.
#include "common.h"

namespace sdpa {
namespace {

// Philox4x32 round multipliers and Weyl key increments (Salmon et al., SC 2011).
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    // one 32 x 32 -> 64-bit product per multiplier (a single v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c[0], p1 = (uint64_t)kPhiloxM1 * c[2];
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__global__ __launch_bounds__(256) void dropout_mask_kernel(DropoutParams p, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int64_t row = idx / p.keep_words;
  const int64_t w = idx % p.keep_words;
  const uint32_t bh = (uint32_t)(row / p.Tq), i = (uint32_t)(row % p.Tq);
  const uint32_t k0 = (uint32_t)p.seed, k1 = (uint32_t)(p.seed >> 32);
  uint32_t word = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int64_t j0 = 32 * w + 8 * c;          // first key of this Philox block
    uint32_t x[4] = {(uint32_t)(j0 / 8), i, bh, p.step};
    philox4x32_10(x, k0, k1);
#pragma unroll
    for (int h = 0; h < 4; ++h) {               // keys 2 h (low half) and 2 h + 1 (high half)
      word |= (uint32_t)((x[h] & 0xFFFFu) >= p.thresh) << (8 * c + 2 * h);
      word |= (uint32_t)((x[h] >> 16) >= p.thresh) << (8 * c + 2 * h + 1);
    }
  }
  // only a row's last word can reach past Tkv: clear those bits once
  const int64_t valid = p.Tkv - 32 * w;
  if (valid < 32) word &= valid <= 0 ? 0u : ((1u << valid) - 1u);
  p.keep[idx] = word;
}

}  // namespace

hipError_t launch_dropout_mask(const DropoutParams& p, hipStream_t s) {
  const int64_t total = p.B * p.Hq * p.Tq * p.keep_words;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, total);
  return hipGetLastError();
}

}  // namespace sdpa
