/*
 * sdpa.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product-attention library.
 *
 *   O = softmax(Q . K^T * scale + B) . V
 *
 * computed without ever writing the T_q x T_kv score matrix, where the
 * additive bias B is one of
 *   - none;
 *   - a causal or sliding-window mask (optionally offset);
 *   - a caller-supplied additive (float) or boolean tensor, broadcast over
 *     [B, Hq, T_q, T_kv] through strides;
 *   - SAM-style decomposed relative position:
 *       B[i, j] = term_h[i, row(j)] + term_w[i, col(j)].
 *
 * Sources (the pages that define the operation):
 *   [Axon PR 650] elixir-nx/axon "Axon.Layers.scaled_dot_product_attention/4",
 *       description: softmax(Q . K^T * scale + mask) . V over rank-4 inputs;
 *       bshd (default) or bhsd axes; scale defaults to 1/sqrt(head_dim);
 *       masks causal, {causal, offset}, {sliding_window, w[, offset]} or a
 *       runtime boolean/float tensor; grouped/multi-query attention by
 *       repeating KV heads.  Review comment on the diff: the output comes
 *       back in the caller's layout, and the contraction should use the
 *       right axes instead of transposing the inputs.
 *   [mlx-examples issue 1451] "segment_anything: fuse attention with
 *       mx.fast.scaled_dot_product_attention", body: SAM's attention blocks,
 *       the add_decomposed_rel_pos bias, and the additive mask broadcast to
 *       [B, N, T_q, T_kv].
 *   [Candle PR 3280] "feat(metal): SDPA with Relative Positional Embeddings
 *       & LayerNorm Stability", Key Changes: a rel-pos attention kernel that
 *       injects per-query term_h / term_w biases into the scores; SDPA for
 *       head_dim 16.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates or frees device memory; scratch space comes in
 *     through `workspace`.
 *   - Dense tensors only.  Layout SDPA_BHSD stores [B, H, T, D] row-major;
 *     SDPA_BSHD stores [B, T, H, D] row-major.  Q and O use Hq heads, K and V
 *     use Hkv heads.  No input is transposed or copied.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues kernels on that stream and returns; it never synchronises.
 *     The backward calls may also run one kernel on a second stream of the
 *     device, forked from and joined back into `stream` with events (tuning
 *     key "bwd_concurrent"), so ordering against `stream` is unchanged.
 *   - Status codes: SDPA_OK (0) or a negative sdpa_status.  Argument errors
 *     are detected before any HIP call is made, so they leave every output
 *     untouched and need no GPU.  sdpa_last_error() gives a thread-local
 *     message for the most recent failing call on the calling thread.
 *   - Calls are thread-safe and deterministic (no atomics in reductions; the
 *     same inputs give bitwise-identical outputs on the same device).  The
 *     process-wide tuning knobs (sdpa_set_tuning) are read once per call, so
 *     one call's route, split count and workspace check always agree; a size
 *     query and the call it sizes see the same knobs unless another thread
 *     changes them in between, and then the call returns SDPA_ERR_WORKSPACE
 *     rather than overrun a short workspace.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_INVALID = -1,      /* null pointer, non-positive size, inconsistent shapes   */
  SDPA_ERR_UNSUPPORTED = -2,  /* valid request that the library does not implement         */
  SDPA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than sdpa_workspace_size() */
  SDPA_ERR_HIP = -4           /* a kernel launch failed; see sdpa_last_error()           */
} sdpa_status;

/* Element types.  SDPA_F16 inputs ([mlx-examples issue 1451], body: fp16
 * together with the fused kernel, and the question of the additive rel-pos
 * bias in fp16) run on the same kernels as SDPA_BF16; scores, the rel-pos
 * bias and the softmax statistics stay in fp32 whatever the input type. */
typedef enum sdpa_dtype { SDPA_F32 = 0, SDPA_BF16 = 1, SDPA_F16 = 2 } sdpa_dtype;

/* [Axon PR 650], description: `:axes` is :bshd (default) or :bhsd. */
typedef enum sdpa_layout { SDPA_BSHD = 0, SDPA_BHSD = 1 } sdpa_layout;

/* [Axon PR 650], description: the `:mask` option family;
 * [mlx-examples issue 1451], body: an additive array broadcast to [B, N, T_q, T_kv]. */
typedef enum sdpa_mask_kind {
  SDPA_MASK_NONE = 0,
  SDPA_MASK_CAUSAL = 1,    /* key j allowed for query i iff j <= i + offset                 */
  SDPA_MASK_SLIDING = 2,   /* allowed iff i + offset - window < j <= i + offset (w keys)     */
  SDPA_MASK_ADDITIVE = 3,  /* B[b,h,i,j] = data[...] (F32 or BF16), added to the scores      */
  SDPA_MASK_BOOL = 4       /* uint8: nonzero = attend, zero = masked (-inf)                   */
} sdpa_mask_kind;

typedef struct sdpa_mask {
  int32_t kind;            /* sdpa_mask_kind                                                  */
  int32_t data_dtype;      /* ADDITIVE: SDPA_F32 or SDPA_BF16; ignored otherwise              */
  int64_t offset;          /* CAUSAL / SLIDING diagonal offset (0 = top-left aligned)         */
  int64_t window;          /* SLIDING: number of keys, >= 1                                   */
  const void* data;        /* ADDITIVE / BOOL: device pointer; NULL otherwise                 */
  int64_t stride[4];       /* ADDITIVE / BOOL: element strides over [B, Hq, T_q, T_kv];
                              0 broadcasts that axis                                          */
} sdpa_mask;

/*
 * Bytes of device workspace that sdpa_fwd (relpos = 0) or sdpa_relpos_fwd
 * (relpos = 1; then Tq = Tkv = grid_h * grid_w and Hkv = Hq) needs for a call
 * with this input dtype, these sizes and this scale (NaN = 1/sqrt(D)), under
 * the current tuning knobs.  The answer follows the route the call takes:
 * split-KV partials for few-query head_dim-16 calls and for 16-bit
 * head_dim-64 / 128 calls whose query blocks leave most of the GPU idle
 * against a long key range (decode shapes), fp32 term arrays for a rel-pos
 * call that cannot form its terms inside the attention kernel, and 0 when the
 * call needs none (e.g. every fused rel-pos route, SAM ViT-B's 64 x 64 global
 * grid included).  The mask is not an argument: the answer is the unmasked
 * call's, which is also enough for any mask (a head_dim-64 / 128 call with a
 * tensor mask runs unsplit and leaves the workspace unused).  Pure host
 * arithmetic: no HIP call.
 * Returns (size_t)-1 for invalid sizes or dtype.
 */
size_t sdpa_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv,
                           int64_t D, float scale, int relpos, int64_t grid_h, int64_t grid_w);

/*
 * Fused attention with an optional mask.  [Axon PR 650], description.
 *   q [B, Hq, Tq, D] / [B, Tq, Hq, D], k and v [.., Hkv, Tkv, ..], o like q.
 *   dtype      element type of q, k, v (SDPA_F32, SDPA_BF16 or SDPA_F16).
 *   out_dtype  element type of o: dtype, or SDPA_F32 for unrounded output.
 *   Hq % Hkv == 0; query head h reads KV head h / (Hq / Hkv).
 *   D          head_dim: 16, 32, 64 or 128 (16-bit types); 1..128 (SDPA_F32).
 *   scale      multiplies Q.K^T; NaN selects 1/sqrt(D).
 *   mask       NULL or &sdpa_mask{kind = NONE} for no mask.
 *   lse        optional [B, Hq, Tq] fp32 log-sum-exp of each score row
 *              (natural log; -inf for a row with no allowed key); NULL skips it.
 *   Rows with no allowed key produce O = 0.
 *   workspace  device scratch of at least sdpa_workspace_size(dtype, ..., scale, 0, 0, 0)
 *              bytes (may be NULL when that size is 0).
 */
int sdpa_fwd(const void* q, const void* k, const void* v, void* o,
             int dtype, int out_dtype, int layout,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D,
             float scale, const sdpa_mask* mask, float* lse,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and kernels as sdpa_fwd, minus the workspace: the
 * split-KV partials of the few-query routes live in a fixed 8 MiB device
 * array inside the library (one copy per GPU, held until the process ends).
 * The call allocates and frees nothing; its first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress).  Where the automatic
 * split count's partials would exceed 8 MiB the call runs with the largest
 * count that fits (results then equal sdpa_fwd's up to rounding, not
 * bitwise); a forced "num_splits" whose partials exceed 8 MiB returns
 * SDPA_ERR_UNSUPPORTED.  Every call on one GPU shares that GPU's array and leaves the
 * last call's partials in it: calls that overlap on one GPU (concurrent
 * streams or threads) race on it and must be serialised by the caller.
 */
int sdpa_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                     int dtype, int out_dtype, int layout,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D,
                     float scale, const sdpa_mask* mask, float* lse, void* stream);

/*
 * Decomposed rel-pos terms of SAM's attention ([mlx-examples issue 1451],
 * body: add_decomposed_rel_pos; [Candle PR 3280], Key Changes: term_h/term_w):
 *   term_h[b,h,i,y] = sum_c q[b,h,i,c] * rel_pos_h[row(i) - y + grid_h - 1, c]
 *   term_w[b,h,i,x] = sum_c q[b,h,i,c] * rel_pos_w[col(i) - x + grid_w - 1, c]
 * with row(i) = i / grid_w, col(i) = i % grid_w and the UNSCALED query.
 *   q          [B, H, T, D] or [B, T, H, D] with T = grid_h * grid_w, in dtype.
 *   rel_pos_h  [2*grid_h - 1, D] in dtype; rel_pos_w [2*grid_w - 1, D].
 *   term_h     [B, H, T, grid_h] fp32 output; term_w [B, H, T, grid_w] fp32.
 *   Products accumulate in fp32.
 */
int relpos_terms(const void* q, int dtype, int layout,
                 int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                 const void* rel_pos_h, const void* rel_pos_w,
                 float* term_h, float* term_w, void* stream);

/*
 * Fused attention with the decomposed rel-pos bias, never materialising a
 * T x T array ([Candle PR 3280], Key Changes: the bias is injected from the
 * term rows; [mlx-examples issue 1451], body: SAM's image-encoder block).
 *   Self-attention on a grid_h x grid_w token grid: Tq = Tkv = grid_h*grid_w,
 *   Hq = Hkv = H.  Scores are scale * q.k + term_h[i,row(j)] + term_w[i,col(j)]
 *   (the bias is not scaled).  Other arguments as in sdpa_fwd.
 *   workspace  at least sdpa_workspace_size(dtype, B, H, H, T, T, D, scale, 1, grid_h,
 *              grid_w) bytes.  A call that forms the terms inside the attention
 *              kernel (sdpa_relpos_fused) does not touch it: NULL / 0 is accepted.
 */
int sdpa_relpos_fwd(const void* q, const void* k, const void* v, void* o,
                    int dtype, int out_dtype, int layout,
                    int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                    const void* rel_pos_h, const void* rel_pos_w,
                    float scale, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * 1 if sdpa_relpos_fwd with these parameters forms the rel-pos terms inside
 * the attention kernel (a single kernel launch, no term arrays), 0 if it
 * first runs relpos_terms into the workspace.  Holds for a positive finite
 * scale; any other scale always takes the two-launch route.  Pure host logic,
 * no HIP call.
 */
int sdpa_relpos_fused(int dtype, int64_t D, int64_t grid_h, int64_t grid_w);

/* Static description of a status code. */
const char* sdpa_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* sdpa_last_error(void);

/*
 * Name of the attention kernel that the last successful sdpa_fwd /
 * sdpa_relpos_fwd call on this thread launched (its dominant kernel; a
 * split-KV combine or a separate relpos_terms launch is not named), or "" if
 * none yet.  Static string, never freed.  For profiling and benchmarks.
 */
const char* sdpa_last_kernel(void);

/*
 * Process-wide tuning knobs (tests and benchmarks), each an int64:
 *   "num_splits"   split-KV chunk count for sdpa_fwd; 0 = automatic (default),
 *                  1 = never split, n > 1 = n chunks when the kernel supports it
 *                  (head_dim 16 with <= 8 queries: chunks of >= 64 keys, at most
 *                  1024; 16-bit head_dim 64 / 128 with no mask or a causal /
 *                  sliding mask: chunks of >= 32 keys, at most 64).
 *   "split_halves" 1 (default) = for head_dim 64 with few query rows, each
 *                  workgroup splits the key range between its waves and merges
 *                  the halves; 0 = always one key range per wave.
 *   "split_wide"   1 (default) = of those, shapes whose query rows fill the
 *                  CUs in workgroups of 192 rows run on 12-wave workgroups
 *                  (six 32-row query blocks x two key halves); 2 = every such
 *                  shape runs on them; 0 = always the 4-wave workgroups.
 *   "tiled"        1 (default) = bf16 head_dim 64 / 128 attention with no mask
 *                  or a causal / sliding mask runs on the double-buffered
 *                  kernel; 0 = on the general MFMA kernel.
 *   "relpos_fused" 1 (default) = sdpa_relpos_fwd forms the rel-pos terms
 *                  inside the attention kernel where the grid allows it;
 *                  0 = always run relpos_terms into the workspace first.
 *   "relpos_mfma"  1 (default) = relpos_terms (also inside sdpa_relpos_bwd)
 *                  forms 16-bit inputs' terms on the matrix cores where
 *                  head_dim and the grid allow it; 0 = on the vector ALUs.
 *   "relpos_bwd_mfma" 1 (default) = sdpa_relpos_bwd forms the tables'
 *                  gradients and the tables' part of dq on the matrix cores
 *                  where the grid allows it (both sides <= 64); 0 = on the
 *                  vector ALUs.
 *   "bwd_concurrent" 1 (default) = where the grid of the dK/dV or the dQ
 *                  kernel leaves at least a tenth of its last round of
 *                  resident workgroups empty, the backward calls run the two
 *                  side by side: dQ on a second stream of the device (created once
 *                  per device, default priority; a call on a stream that is
 *                  being captured into a graph, or that belongs to another
 *                  device than the calling thread's current one, keeps both
 *                  kernels on it),
 *                  followed there by the rel-pos
 *                  tables' gradients, forked from and joined back into the
 *                  caller's stream with events, so later work on the
 *                  caller's stream still sees every gradient.  The
 *                  results are the same bit for bit.  Calls on several
 *                  streams of one device share its second stream, so their
 *                  dQ kernels run in the order the calls were made.
 *                  0 = both on the caller's stream, one after the other.
 *   "generic_waves" 0 (default) = the vector-ALU kernel (fp32, and shapes no
 *                  matrix-core kernel takes) splits each 64-row block's keys
 *                  over 4 waves when the launch has fewer blocks than the GPU
 *                  has compute units and head_dim <= 32; 1 = always one wave.
 * Returns SDPA_OK, or SDPA_ERR_INVALID for an unknown key or bad value.
 * sdpa_workspace_size answers for the knobs in force when it is called.
 */
int sdpa_set_tuning(const char* key, int64_t value);

/* ---------------------------------------------------------------------------
 * Training path.  [Axon PR 650], description: `:dropout_rate` drops attention
 * probabilities in :train mode, with a PRNG key that the graph layer threads
 * across steps; `:return_attention_weights`; and the gradients a training
 * step needs.
 *
 * Dropout works on keep bits: one bit per score element, packed as uint32
 * words [B, Hq, Tq, ceil(Tkv / 32)] (bit j % 32 of word j / 32 keeps score
 * (b, h, i, j); bits past Tkv are zero).  A dropped weight contributes nothing
 * to O; a kept one is multiplied by 65536 / (65536 - thresh), where
 * thresh = floor(rate * 65536 + 0.5) clamped to 65535, so the kept weights are
 * unbiased.  The row normalisation and lse are those of the undropped scores.
 * ------------------------------------------------------------------------- */

/*
 * Keep bits from the counter-based generator Philox4x32-10 (Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011):
 * score (b, h, i, j) takes the 16-bit half j % 8 (low half of word
 * (j % 8) / 2 first) of Philox(counter = (j / 8, i, b * Hq + h, step),
 * key = (seed low 32 bits, seed high 32 bits)) and is kept iff that half
 * >= thresh.  The same (seed, step) always gives the same bits; a training
 * loop advances `step` (or the seed) every call.
 *   keep   device output, B * Hq * Tq * ceil(Tkv / 32) uint32 words.
 *   rate   in [0, 1).  B * Hq, Tq and Tkv must fit in 31 bits.
 */
int sdpa_dropout_mask(uint64_t seed, uint32_t step, float rate, int64_t B, int64_t Hq, int64_t Tq, int64_t Tkv,
                      uint32_t* keep, void* stream);

/*
 * Fused attention with attention dropout: O = (W * Z) . V, with W the softmax
 * weights of sdpa_fwd and Z = keep bit * 65536 / (65536 - thresh).  Arguments
 * as in sdpa_fwd, plus the keep bits (required, device) and the rate that
 * produced them.  lse (optional) is that of the undropped scores.
 * Runs on the double-buffered matrix-core kernel (bf16 / fp16, head_dim
 * 64 / 128, no mask or a causal / sliding mask, positive scale), else on the
 * general matrix-core kernel (bf16, head_dim 64 / 128, positive scale), else
 * on the generic kernel; the workspace is not used (may be NULL).
 */
int sdpa_fwd_dropout(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype, int layout,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
                     const sdpa_mask* mask, const uint32_t* keep, float rate, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace sdpa_relpos_fwd_dropout needs: both fp32 term
 * arrays, [B, H, T, grid_h] and [B, H, T, grid_w], each 256-byte aligned
 * ((size_t)-1 for invalid sizes).  Pure host arithmetic.
 */
size_t sdpa_relpos_fwd_dropout_workspace_size(int64_t B, int64_t H, int64_t grid_h, int64_t grid_w);

/*
 * sdpa_relpos_fwd with attention dropout ([Axon PR 650], description:
 * `:dropout_rate` in :train mode, applied to the weights; [mlx-examples issue
 * 1451], body: SAM's rel-pos bias): O = (W * Z) . V with W the softmax of
 * scale * q.k + term_h[i,row(j)] + term_w[i,col(j)] and Z as in
 * sdpa_fwd_dropout.  keep holds B * H * T * ceil(T / 32) words from
 * sdpa_dropout_mask(seed, step, rate, B, H, T, T, ...); lse is that of the
 * undropped scores.  relpos_terms always runs first into the workspace
 * (sdpa_relpos_fwd_dropout_workspace_size bytes); the attention then runs on
 * the double-buffered matrix-core kernel (bf16 / fp16, head_dim 64 / 128,
 * grid_w a multiple of 4, positive scale), else on the generic kernel.
 */
int sdpa_relpos_fwd_dropout(const void* q, const void* k, const void* v, void* o, int dtype, int out_dtype,
                            int layout, int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                            const void* rel_pos_h, const void* rel_pos_w, float scale, const uint32_t* keep,
                            float rate, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace sdpa_bwd needs ((size_t)-1 for invalid sizes). */
size_t sdpa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Tq);

/*
 * Gradients of attention: for a loss with upstream gradient dout = dL/dO,
 *   dv = (W * Z)^T . dout            (summed over the query heads sharing a KV head)
 *   dW = (dout . v^T) * Z,   dS = W * (dW - rowsum(dout * o))
 *   dq = scale * dS . k,     dk = scale * dS^T . q   (summed likewise)
 * with W rebuilt from q, k, the mask and the forward pass's lse (no T x T
 * array is stored).  Rows with no allowed key get zero gradients.
 *   q, k, v, o, dout  as in sdpa_fwd (o and dout shaped like q); o in o_dtype
 *                     (dtype or SDPA_F32), the forward pass's output.
 *   lse               [B, Hq, Tq] fp32 from the forward pass (required).
 *   dq, dk, dv        outputs shaped like q, k, v, in grad_dtype (dtype or SDPA_F32);
 *                     fully overwritten.
 *   mask              as in sdpa_fwd; keep / rate as in sdpa_fwd_dropout
 *                     (keep NULL = no dropout).
 *   workspace         at least sdpa_bwd_workspace_size(B, Hq, Tq) bytes.
 * Built for bf16 / fp16 inputs with head_dim 32, 64 or 128 and 16-byte aligned
 * tensors (SDPA_ERR_UNSUPPORTED otherwise).  Deterministic: no atomics.
 */
int sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int dtype, int o_dtype, int grad_dtype, int layout,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tkv, int64_t D, float scale,
             const sdpa_mask* mask, const uint32_t* keep, float rate, void* workspace, size_t workspace_bytes,
             void* stream);

/* Bytes of device workspace sdpa_relpos_bwd needs ((size_t)-1 for invalid sizes). */
size_t sdpa_relpos_bwd_workspace_size(int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D);

/*
 * Gradients of the rel-pos attention of sdpa_relpos_fwd ([mlx-examples issue
 * 1451], body: SAM's add_decomposed_rel_pos; [Candle PR 3280], Key Changes:
 * term_h / term_w): as sdpa_bwd for the bias B[i, j] = term_h[i, row(j)] +
 * term_w[i, col(j)], which also depends on q and on the tables:
 *   dq_i += sum_y dT_h[i, y] rel_pos_h[row(i) - y + grid_h - 1]
 *         + sum_x dT_w[i, x] rel_pos_w[col(i) - x + grid_w - 1],
 *   d_rel_pos_h[t] = sum over (b, h, i, y) with row(i) - y + grid_h - 1 = t of dT_h[i, y] q_i
 *   (d_rel_pos_w alike), with dT_h[i, y] the sum of dS[i, j] over the keys j of
 *   grid row y and dT_w[i, x] over grid column x.
 *   q .. lse, dq, dk, dv   as in sdpa_bwd with Hq = Hkv = H and Tq = Tkv = grid_h * grid_w.
 *   rel_pos_h, rel_pos_w   the tables of the forward call, in dtype.
 *   d_rel_pos_h            [2 grid_h - 1, D] fp32 output; d_rel_pos_w [2 grid_w - 1, D].
 *   workspace              at least sdpa_relpos_bwd_workspace_size(B, H, grid_h, grid_w, D) bytes.
 * Built for bf16 / fp16, head_dim 32, 64 or 128, grid_w >= 4 and grid_h + grid_w
 * <= 128 (SAM's 14 x 14 windows and 64 x 64 global grid).  With dropout see
 * sdpa_relpos_bwd_dropout.  Deterministic: no atomics.
 */
int sdpa_relpos_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, float* d_rel_pos_h, float* d_rel_pos_w, int dtype, int o_dtype,
                    int grad_dtype, int layout, int64_t B, int64_t H, int64_t grid_h, int64_t grid_w, int64_t D,
                    const void* rel_pos_h, const void* rel_pos_w, float scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * sdpa_relpos_bwd for the forward pass of sdpa_relpos_fwd_dropout: the same
 * gradients with the weights that multiply V scaled by Z (dW = (dout . v^T)
 * * Z as in sdpa_bwd), so dS, the term gradients and the tables' gradients
 * carry the dropout.  keep (required) and rate as given to the forward call;
 * other arguments, limits and workspace as in sdpa_relpos_bwd.
 */
int sdpa_relpos_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* d_rel_pos_h, float* d_rel_pos_w,
                            int dtype, int o_dtype, int grad_dtype, int layout, int64_t B, int64_t H, int64_t grid_h,
                            int64_t grid_w, int64_t D, const void* rel_pos_h, const void* rel_pos_w, float scale,
                            const uint32_t* keep, float rate, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * The attention weights (`:return_attention_weights`): weights[b, h, i, j] =
 * exp(scale * q_i . k_j + bias_ij - lse_i) * Z_ij, i.e. the weights that
 * multiply V in the forward pass that produced lse (Z = 1 without keep bits).
 *   weights  device output [B, Hq, Tq, Tkv] fp32 (a T x T array: a debug output).
 *   lse      [B, Hq, Tq] fp32 from sdpa_fwd / sdpa_fwd_dropout on the same inputs.
 * Any dtype and head_dim up to 128; B * Hq and Tq / 64 must stay below 65536.
 * 16-bit inputs at head_dim 32 / 64 / 128 with 16-byte aligned Q and K and
 * strides in multiples of 8 elements run on the matrix cores; other calls on
 * the vector ALUs (same results up to fp32 summation order).
 */
int sdpa_attention_weights(const void* q, const void* k, int dtype, int layout, int64_t B, int64_t Hq, int64_t Hkv,
                           int64_t Tq, int64_t Tkv, int64_t D, float scale, const sdpa_mask* mask, const float* lse,
                           const uint32_t* keep, float rate, float* weights, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
