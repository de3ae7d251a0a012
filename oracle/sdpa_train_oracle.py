"""fp64 oracle for the training path of attention (test infrastructure only).

Covers what [Axon PR 650] elixir-nx/axon "Axon.Layers.scaled_dot_product_attention/4"
lists beyond the inference forward pass (description): attention-probability
dropout in :train mode with a PRNG key that the graph layer threads from step
to step, `:return_attention_weights`, and -- implied by training -- the
gradients of the attention with respect to Q, K, V (and, for SAM's decomposed
rel-pos bias of [mlx-examples issue 1451] "segment_anything: fuse attention
with mx.fast.scaled_dot_product_attention", body, the two tables).

Everything is materialised and written as the plain definition; only tests,
the smoke check and the CPU-baseline leg of the benchmark may use it.  It
shares no code with the HIP library.

Readings where the pages leave a step open (listed with the others in the
design notes):

* Dropout acts on the softmax weights after normalisation and before the
  product with V (the diff in the review thread applies
  maybe_attention_dropout to the weights, then contracts them with V):
  W~ = W * Z with Z = keep / (1 - rate_eff).  The row log-sum-exp is that of
  the undropped scores.
* The PRNG is Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator: the
  64-bit seed is the key, and the counter of score element (b, h, i, j) is
  (j // 8, i, b * Hq + h, step).  `step` is the per-step counter the key
  threading advances.  The four 32-bit outputs give eight 16-bit numbers,
  u = half (j % 8) (low half of word (j % 8) // 2 first).  Element kept iff
  u >= thresh, thresh = floor(rate * 65536 + 0.5) clamped to 65535, so the
  effective rate is thresh / 65536 and Z = 65536 / (65536 - thresh) for kept
  elements (unbiased: E[Z] = 1 exactly).
* `:return_attention_weights` returns the weights that multiply V, i.e. W~
  in :train mode with dropout and the softmax W otherwise.
* Gradients are those of O = W~ . V with W = softmax(scale * Q.K^T + B);
  rows with no allowed key have zero gradient.  With grouped-query attention
  the K/V gradients sum over the query heads that share a KV head.
"""
from __future__ import annotations

import numpy as np

from .sdpa_oracle import (_bias_rows, _prepare, from_bhsd, kv_head_of,
                          softmax_rows, to_bhsd)

__all__ = ["philox4x32_10", "dropout_threshold", "dropout_keep", "pack_keep_words",
           "unpack_keep_words", "sdpa_train_fwd", "attention_weights", "sdpa_bwd"]

_M32 = 0xFFFFFFFF
# Philox4x32 round multipliers and Weyl key increments (Salmon et al., SC 2011, Table 2 / Section 3.3).
_PHILOX_M0, _PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
_PHILOX_W0, _PHILOX_W1 = 0x9E3779B9, 0xBB67AE85


# ------------------------------------------------------------------ Philox ---
def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds on arrays of counters.

    ctr: 4 arrays (or ints) of 32-bit counter words (c0, c1, c2, c3);
    key: 2 arrays (or ints) of 32-bit key words (k0, k1).
    One round (Salmon et al., SC 2011, Section 3.3): with the two products
    M0 * c0 and M1 * c2 split into high and low 32-bit halves,
        (c0, c1, c2, c3) <- (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
    and the key is bumped by the Weyl constants (W0, W1) between rounds.
    Returns the 4 output words as uint64 arrays holding 32-bit values.
    """
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(_M32) for x in ctr]
    k0, k1 = (np.asarray(x, dtype=np.uint64) & np.uint64(_M32) for x in key)
    m0, m1 = np.uint64(_PHILOX_M0), np.uint64(_PHILOX_M1)
    lo_mask, sh = np.uint64(_M32), np.uint64(32)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(_PHILOX_W0)) & lo_mask
            k1 = (k1 + np.uint64(_PHILOX_W1)) & lo_mask
        p0 = m0 * c[0]                   # < 2**64: exact in uint64
        p1 = m1 * c[2]
        c = [(p1 >> sh) ^ c[1] ^ k0, p1 & lo_mask, (p0 >> sh) ^ c[3] ^ k1, p0 & lo_mask]
    return c


def dropout_threshold(rate):
    """(thresh, keep_scale): keep iff a 16-bit uniform u >= thresh; kept weights x keep_scale."""
    rate = float(rate)
    if not (0.0 <= rate < 1.0):
        raise ValueError("dropout rate must be in [0, 1)")
    thresh = min(65535, int(np.floor(rate * 65536.0 + 0.5)))
    return thresh, 65536.0 / (65536.0 - thresh)


def dropout_keep(seed, step, rate, B, Hq, Tq, Tkv):
    """Boolean keep mask [B, Hq, Tq, Tkv] of the dropout reading stated in the header."""
    thresh, _ = dropout_threshold(rate)
    seed = int(seed) & ((1 << 64) - 1)
    ng = (Tkv + 7) // 8
    b, h, i, jg = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Tq), np.arange(ng), indexing="ij")
    words = philox4x32_10((jg, i, b * Hq + h, np.full(jg.shape, int(step) & _M32)),
                          (seed & _M32, seed >> 32))
    halves = []
    for w in words:                      # word e // 2, low half first
        halves.append(w & np.uint64(0xFFFF))
        halves.append(w >> np.uint64(16))
    u = np.stack(halves, axis=-1).reshape(B, Hq, Tq, ng * 8)[..., :Tkv]
    return u >= np.uint64(thresh)


def pack_keep_words(keep):
    """[.., Tkv] bool -> [.., ceil(Tkv / 32)] uint32, bit j % 32 of word j // 32 (zero beyond Tkv)."""
    keep = np.asarray(keep, dtype=bool)
    Tkv = keep.shape[-1]
    nw = (Tkv + 31) // 32
    padded = np.zeros(keep.shape[:-1] + (nw * 32,), dtype=np.uint64)
    padded[..., :Tkv] = keep
    bits = padded.reshape(keep.shape[:-1] + (nw, 32)) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=-1).astype(np.uint32)


def unpack_keep_words(words, Tkv):
    """Inverse of pack_keep_words."""
    w = np.asarray(words, dtype=np.uint64)
    bits = (w[..., None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(w.shape[:-1] + (w.shape[-1] * 32,))[..., :Tkv].astype(bool)


def _zfactor(keep, rate, shape):
    if keep is None:
        return None
    _, kscale = dropout_threshold(rate)
    keep = np.broadcast_to(np.asarray(keep, dtype=bool), shape)
    return np.where(keep, kscale, 0.0)


# -------------------------------------------------------------- forward ---
def _weights(q, k, v, dims, scale, mask, rel_pos, terms):
    """Per (b, h): the softmax weights W [Tq, Tkv] of the definition."""
    B, Hq, Hkv, Tq, Tkv, D = dims
    rows = np.arange(Tq)
    W = np.zeros((B, Hq, Tq, Tkv))
    lse = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            z = scale * (q[b, h] @ k[b, g].T) + _bias_rows(b, h, rows, dims, mask, rel_pos, terms)
            W[b, h], lse[b, h] = softmax_rows(z)
    return W, lse


def sdpa_train_fwd(q, k, v, *, layout="bhsd", scale=None, mask=None, rel_pos=None, keep=None, rate=0.0):
    """O = (W * Z) . V with W the softmax weights, Z the dropout factor (keep [B,Hq,Tq,Tkv] bool or None).

    Returns {"o": O in `layout`, "lse": [B,Hq,Tq] of the undropped scores}.
    """
    q, k, v, dims, scale, terms = _prepare(q, k, v, layout, scale, rel_pos)
    B, Hq, Hkv, Tq, Tkv, D = dims
    W, lse = _weights(q, k, v, dims, scale, mask, rel_pos, terms)
    Z = _zfactor(keep, rate, W.shape)
    Wt = W if Z is None else W * Z
    o = np.zeros((B, Hq, Tq, D))
    for b in range(B):
        for h in range(Hq):
            o[b, h] = Wt[b, h] @ v[b, kv_head_of(h, Hq, Hkv)]
    return {"o": from_bhsd(o, layout), "lse": lse}


def attention_weights(q, k, *, layout="bhsd", scale=None, mask=None, keep=None, rate=0.0):
    """[B, Hq, Tq, Tkv]: the weights that multiply V (W, or W * Z with dropout)."""
    v = np.zeros_like(np.asarray(k, dtype=np.float64))
    q, k, v, dims, scale, terms = _prepare(q, k, v, layout, scale, None)
    W, _ = _weights(q, k, v, dims, scale, mask, None, None)
    Z = _zfactor(keep, rate, W.shape)
    return W if Z is None else W * Z


# ------------------------------------------------------------- backward ---
def sdpa_bwd(q, k, v, dout, *, layout="bhsd", scale=None, mask=None, rel_pos=None, keep=None, rate=0.0):
    """Gradients of L = sum(O * dout) for O = (W * Z) . V, W = softmax(scale Q.K^T + B).

    The chain rule written out per (b, h), with Zs the scores and W their softmax:
        dV   += (W * Z)^T . dO                 (summed over the heads sharing the KV head)
        dW    = (dO . V^T) * Z
        dZs   = W * (dW - rowsum(W * dW))      (Jacobian of the row softmax)
        dQ    = scale * dZs . K
        dK   += scale * dZs^T . Q
    and for the decomposed rel-pos bias B[i, j] = term_h[i, row(j)] + term_w[i, col(j)]
    with term_h[i, y] = q_i . Rh[row(i) - y + gh - 1] (likewise w):
        dterm_h[i, y] = sum over keys j in grid row y of dZs[i, j]   (dterm_w over grid column x)
        dQ_i         += sum_y dterm_h[i, y] Rh[row(i) - y + gh - 1] + sum_x dterm_w[i, x] Rw[col(i) - x + gw - 1]
        dRh[row(i) - y + gh - 1] += dterm_h[i, y] q_i   (over every b, h, i, y; likewise dRw)
    Returns {"dq", "dk", "dv"} in `layout` (float64), plus "drel_pos_h", "drel_pos_w" with rel_pos.
    """
    q, k, v, dims, scale, terms = _prepare(q, k, v, layout, scale, rel_pos)
    B, Hq, Hkv, Tq, Tkv, D = dims
    do = to_bhsd(np.asarray(dout, dtype=np.float64), layout)
    W, _ = _weights(q, k, v, dims, scale, mask, rel_pos, terms)
    Z = _zfactor(keep, rate, W.shape)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    out = {}
    if rel_pos is not None:
        gh, gw = rel_pos["grid"]
        rh = np.asarray(rel_pos["rel_pos_h"], dtype=np.float64)
        rw = np.asarray(rel_pos["rel_pos_w"], dtype=np.float64)
        drh = np.zeros_like(rh)
        drw = np.zeros_like(rw)
        t = np.arange(Tq)
        row, col = t // gw, t % gw
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            Wb = W[b, h]
            Wt = Wb if Z is None else Wb * Z[b, h]
            dv[b, g] += Wt.T @ do[b, h]
            dW = do[b, h] @ v[b, g].T
            if Z is not None:
                dW = dW * Z[b, h]
            dZs = Wb * (dW - np.sum(Wb * dW, axis=1, keepdims=True))
            dq[b, h] = scale * (dZs @ k[b, g])
            dk[b, g] += scale * (dZs.T @ q[b, h])
            if rel_pos is not None:
                dth = dZs.reshape(Tq, gh, gw).sum(axis=2)          # [Tq, gh]
                dtw = dZs.reshape(Tq, gh, gw).sum(axis=1)          # [Tq, gw]
                for i in range(Tq):
                    ih = row[i] - np.arange(gh) + gh - 1             # table rows, one per y
                    iw = col[i] - np.arange(gw) + gw - 1
                    dq[b, h, i] += dth[i] @ rh[ih] + dtw[i] @ rw[iw]
                    np.add.at(drh, ih, dth[i][:, None] * q[b, h, i][None, :])
                    np.add.at(drw, iw, dtw[i][:, None] * q[b, h, i][None, :])
    out.update({"dq": from_bhsd(dq, layout), "dk": from_bhsd(dk, layout), "dv": from_bhsd(dv, layout)})
    if rel_pos is not None:
        out["drel_pos_h"], out["drel_pos_w"] = drh, drw
    return out
