// Internal interface between the host dispatcher (abi.cpp) and the HIP kernels.
// Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

enum BiasKind : int {
  BIAS_NONE = 0,
  BIAS_CAUSAL = 1,     // j <= i + offset
  BIAS_SLIDING = 2,    // i + offset - window < j <= i + offset
  BIAS_ADDITIVE = 3,   // + data[b,h,i,j] through strides
  BIAS_BOOL = 4,       // data[b,h,i,j] != 0 attends
  BIAS_RELPOS = 5      // + term_h[b,h,i,row(j)] + term_w[b,h,i,col(j)]
};

// Everything a forward kernel needs.  Strides are in elements.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                 // [B, Hq, Tq] or nullptr
  int dtype;                  // SDPA_F32 / SDPA_BF16
  int out_dtype;
  int64_t B, Hq, Hkv, Tq, Tkv, D;
  int64_t q_sb, q_sh, q_st;   // q and o
  int64_t k_sb, k_sh, k_st;   // k and v
  float scale;
  int bias;                   // BiasKind
  int64_t offset, window;     // causal / sliding
  const void* mdata;          // additive / bool data
  int mdtype;                 // additive element type
  int64_t ms[4];              // mask strides over [B, Hq, Tq, Tkv]
  const float* term_h;        // rel-pos terms [B, Hq, Tq, grid_h] fp32
  const float* term_w;        // [B, Hq, Tq, grid_w] fp32
  const void* rel_h;          // rel-pos tables for kernels that form the terms themselves
  const void* rel_w;
  int grid_h, grid_w;
  int relpos_rows_lds;        // generic kernel: term rows staged in LDS (set by its launcher)
  int generic_multiwave;      // generic kernel: key range split over 4 waves on small launches (1) or not (0)
  int num_splits;             // split-KV chunks (1 = no split)
  float* part_o;              // split-KV partial outputs [splits, B, Hq, Tq, D] fp32
  float* part_ml;             // split-KV partial (max, sum) [splits, B, Hq, Tq, 2] fp32
  const uint32_t* keep;       // dropout keep bits [B, Hq, Tq, keep_words] or nullptr (no dropout)
  int64_t keep_words;         // 32-bit words per score row: ceil(Tkv / 32)
  float keep_scale;           // factor of a kept weight: 65536 / (65536 - threshold)
};

// Everything the backward kernels need.  q, o, dout and dq share the q strides;
// k, v, dk and dv share the k strides.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;           // [B, Hq, Tq] natural-log row log-sum-exp of the forward pass
  void* dq;
  void* dk;
  void* dv;
  float* delta;               // workspace [B, Hq, Tq]: rowsum(dout * o)
  int dtype;                  // SDPA_BF16 / SDPA_F16
  int o_dtype;                // element type of o: dtype or SDPA_F32
  int grad_dtype;             // element type of dq, dk, dv: dtype or SDPA_F32
  int64_t B, Hq, Hkv, Tq, Tkv, D;
  int64_t q_sb, q_sh, q_st;
  int64_t k_sb, k_sh, k_st;
  float scale;
  int bias;                   // BiasKind (no rel-pos)
  int64_t offset, window;
  const void* mdata;
  int mdtype;
  int64_t ms[4];
  const uint32_t* keep;
  int64_t keep_words;
  float keep_scale;
  // Decomposed rel-pos (bias = BIAS_RELPOS): the forward terms, the per-query
  // sums of dS over each grid row / column they receive, an fp32 copy of
  // scale * dS . K (the tables' part is added after), and the tables.
  const float* term_h;        // [B, Hq, Tq, grid_h]
  const float* term_w;        // [B, Hq, Tq, grid_w]
  float* dterm_h;             // [B, Hq, Tq, grid_h]
  float* dterm_w;             // [B, Hq, Tq, grid_w]
  float* dq_acc;              // [B, Hq, Tq, D] fp32
  const void* rel_h;          // [2 grid_h - 1, D] in dtype
  const void* rel_w;          // [2 grid_w - 1, D]
  float* drel_h;              // [2 grid_h - 1, D] fp32 output
  float* drel_w;              // [2 grid_w - 1, D] fp32 output
  float* group_h;             // [split_h][grid_h (row r)][grid_h (y)][D] fp32 scratch
  float* group_w;             // [split_w][grid_w (column c)][grid_w (x)][D] fp32 scratch
  int grid_h, grid_w;
  int split_h, split_w;       // query slices of the grouped table products
  int tgrad_mfma;             // table gradients on the matrix cores where the shape allows (1) or not (0)
  int concurrent;             // dK/dV and dQ kernels on two streams, side by side (1) or in sequence (0)
};

// Query slices of a grouped table product: about 512 workgroups in all, each
// with at least 64 queries.  Used by the launcher and the workspace planner.
// Table gradients on the matrix cores: workgroups per table (each keeps a
// [128 x D] fp32 partial sum in the group_h / group_w scratch), and whether a
// shape fits the kernel (tables up to 64 entries wide, a line's dT and q rows
// staged in 64 KB of LDS).
inline int relpos_tgrad_wgs(int64_t B, int64_t H, int64_t gh, int64_t gw) {
  const int64_t items = B * H * (gh > gw ? gh : gw);
  return (int)(items < 256 ? items : 256);
}
inline bool relpos_tgrad_mfma_ok(int64_t B, int64_t H, int64_t gh, int64_t gw, int64_t D) {
  if (gh > 64 || gw > 64 || (D != 32 && D != 64 && D != 128) || B * H > 65535) return false;
  // dT and q are read through descriptors with 32-bit byte offsets
  if (B * H * gh * gw * (gh > gw ? gh : gw) * 4 > 0x7fffffffLL || B * H * gh * gw * D * 2 > 0x7fffffffLL) return false;
  return true;                                  // two staging buffers of at most 64 x (96 x 4 + 128 x 2) bytes
}

inline int relpos_group_splits(int64_t members, int64_t groups) {
  int64_t s = (512 + groups - 1) / groups;
  const int64_t cap = members / 64 > 1 ? members / 64 : 1;
  if (s > cap) s = cap;
  return (int)(s < 1 ? 1 : s);
}

// Dropout keep bits (Philox4x32-10): word [b, h, i, j / 32], bit j % 32.
struct DropoutParams {
  uint64_t seed;
  uint32_t step;
  uint32_t thresh;            // keep iff the element's 16-bit uniform >= thresh
  int64_t B, Hq, Tq, Tkv, keep_words;
  uint32_t* keep;
};

struct TermsParams {
  const void* q;
  int dtype;
  int64_t B, H, T, D;
  int64_t q_sb, q_sh, q_st;
  const void* rel_h;
  const void* rel_w;
  int grid_h, grid_w;
  float* term_h;
  float* term_w;
  int use_mfma;               // 16-bit inputs: products on the matrix cores where the shape allows (1) or not (0)
};

// Split-KV (chunked key range + log-sum-exp merge) is available.
constexpr bool kSplitKvBuilt = true;

// Allocation-free forward: bytes of the fixed per-device scratch array that
// holds the split-KV partials, and its device address on the current device
// (looked up once per device).
constexpr size_t kNoAllocScratchBytes = 8u << 20;
hipError_t noalloc_scratch(void** ptr);

// Launchers: return hipSuccess or the launch error.  Each only enqueues work.
hipError_t launch_generic_fwd(const FwdParams& p, hipStream_t s);
// Rel-pos on the generic kernel: the per-lane term rows (and, fused, the tables) fit its LDS.
bool generic_relpos_supported(const FwdParams& p, bool fused);
hipError_t launch_relpos_terms(const TermsParams& p, hipStream_t s);
hipError_t launch_flash_mfma(const FwdParams& p, hipStream_t s);   // bf16, D in {64, 128}
bool flash_mfma_supports(const FwdParams& p);
hipError_t launch_d16(const FwdParams& p, hipStream_t s);            // bf16, D = 16, head-packed (+ split-KV)
bool d16_supports(const FwdParams& p);
hipError_t launch_split64(const FwdParams& p, hipStream_t s);        // bf16, D = 64, key range split in-workgroup
bool split64_supports(const FwdParams& p);
bool split64_shape_ok(const FwdParams& p);                           // split64_supports without the block-count limit
hipError_t launch_split64w(const FwdParams& p, hipStream_t s);       // as split64, 12-wave workgroups of 192 query rows
bool split64w_supports(const FwdParams& p, bool need_fill);          // need_fill: its workgroups fill the CUs
hipError_t launch_window(const FwdParams& p, hipStream_t s);         // bf16, D = 64, 14 x 14 rel-pos windows, terms in-kernel
bool window_supports(const FwdParams& p);
hipError_t launch_tiled(const FwdParams& p, hipStream_t s);          // bf16, D in {64, 128}, none / causal / sliding
bool tiled_supports(const FwdParams& p);
// Rel-pos terms can be formed inside the MFMA kernel (no term arrays needed).
bool relpos_fused_supported(const FwdParams& p);
hipError_t launch_dropout_mask(const DropoutParams& p, hipStream_t s);
// Backward (16-bit inputs, head_dim 32 / 64 / 128, every bias kind but rel-pos):
// delta, then dK / dV (one workgroup per key block), then dQ (one per query block).
bool bwd_supports(const BwdParams& p);
// Work that needs dq: `tail` runs on s after every kernel of the pass;
// `side_tail` (independent of `tail`'s outputs, and not reading dk / dv) may
// run on a second stream right after the dQ kernel.
using BwdTail = hipError_t (*)(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, hipStream_t s, BwdTail tail = nullptr, BwdTail side_tail = nullptr);
// Rel-pos tail of the backward, in two independent parts:
// dq = dq_acc + the tables' part ...
hipError_t launch_relpos_bwd_dq(const BwdParams& p, hipStream_t s);
// ... and d rel_pos_h / d rel_pos_w.
hipError_t launch_relpos_bwd_tables(const BwdParams& p, hipStream_t s);
// Attention weights [B, Hq, Tq, Tkv] fp32 from the forward pass's lse (any dtype, head_dim <= 128).
hipError_t launch_attn_weights(const FwdParams& p, float* weights, hipStream_t s);
// True if the call runs on the matrix-core weights kernel (16-bit inputs, head_dim 32 / 64 / 128).
bool attn_weights_mfma(const FwdParams& p);

}  // namespace sdpa
