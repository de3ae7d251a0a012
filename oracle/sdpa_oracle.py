"""fp64 oracle for O = softmax(Q.K^T * scale + B) . V  (test infrastructure only).

This module is the plain definition of the operation, written out literally
in numpy float64: the score matrix, the bias matrix and the softmax are all
materialised, exactly as in the unfused attention block the pages describe.
It is slow on purpose and shares no code with the HIP library; only tests,
the smoke check and the benchmark's CPU-baseline leg may use it.

Sources (the three pages this operation is defined by):

* [Axon PR 650] elixir-nx/axon pull request "Axon.Layers.scaled_dot_product_attention/4",
  description: the kernel computes softmax(Q . K^T * scale + mask) . V over
  rank-4 inputs, with `:axes` bshd (default) or bhsd, `:scale` defaulting to
  1/sqrt(head_dim), `:mask` causal / {causal, offset} / {sliding_window, w} /
  {sliding_window, w, offset} / a boolean or float tensor, and grouped-query
  attention by repeating key/value heads.  Review comment on the diff: the
  output is the contraction of the weights with V over the key axis, batched
  over (batch, head), returned in the caller's layout.
* [mlx-examples issue 1451] "segment_anything: fuse attention with
  mx.fast.scaled_dot_product_attention", body: SAM's image-encoder attention
  computes (q * scale) @ k^T, optionally adds add_decomposed_rel_pos's
  relative-position bias, applies softmax over the last axis, then @ v; the
  bias may equally be passed as an additive mask broadcast to [B, N, T_q, T_kv].
* [Candle PR 3280] huggingface/candle pull request "feat(metal): SDPA with
  Relative Positional Embeddings & LayerNorm Stability", Key Changes: the
  rel-pos kernel injects per-query term_h and term_w biases into the scores.

Readings where the pages leave a step open (each is used identically by the
tests; none is pinned by a printed value):

* rel-pos: tokens are laid out row-major on a grid_h x grid_w grid
  (t = row * grid_w + col); term_h[i, y] = q_i . rel_pos_h[row(i) - y + grid_h - 1]
  and term_w[i, x] = q_i . rel_pos_w[col(i) - x + grid_w - 1] with the UNSCALED
  query; bias[i, j] = term_h[i, row(j)] + term_w[i, col(j)], not multiplied
  by scale.  Tables have 2*grid-1 rows and no head axis (shared by all heads).
* causal(offset): key j is allowed for query i iff j <= i + offset.
* sliding(w, offset): allowed iff i + offset - w < j <= i + offset, i.e.
  exactly w keys ending at the diagonal (the window sits on top of causal).
* boolean mask: True means "attend".
* a row with no allowed key has output 0 and log-sum-exp -inf.
* GQA: query head h reads key/value head h // (Hq // Hkv).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["to_bhsd", "from_bhsd", "kv_head_of", "relpos_terms", "relpos_bias",
           "mask_bias", "softmax_rows", "sdpa", "sdpa_rows"]


# ---------------------------------------------------------------- layouts ---
def to_bhsd(x, layout):
    """Return the logical [B, H, T, D] view of a rank-4 array.

    [Axon PR 650], description: `:axes` is :bshd (default) or :bhsd.
    """
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("expected a rank-4 array")
    if layout == "bhsd":
        return x
    if layout == "bshd":
        return x.transpose(0, 2, 1, 3)
    raise ValueError(f"unknown layout {layout!r}")


def from_bhsd(x, layout):
    """Inverse of to_bhsd: [B, H, T, D] back to the caller's layout.

    [Axon PR 650], review comment on the diff: the output is returned in the
    caller's axes.
    """
    if layout == "bhsd":
        return x
    if layout == "bshd":
        return x.transpose(0, 2, 1, 3)
    raise ValueError(f"unknown layout {layout!r}")


def kv_head_of(h, Hq, Hkv):
    """Key/value head read by query head h.

    [Axon PR 650], description: grouped- and multi-query attention repeat the
    key/value heads to match the query heads; repeating each KV head
    Hq // Hkv times in order means query head h uses KV head h // (Hq // Hkv).
    """
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


# ---------------------------------------------------------------- rel-pos ---
def _relpos_index(grid):
    """idx[c_q, c_k] = c_q - c_k + grid - 1: the table row holding the
    embedding of the relative offset between query and key coordinate."""
    c = np.arange(grid)
    return c[:, None] - c[None, :] + grid - 1


def relpos_terms(q_bhsd, rel_pos_h, rel_pos_w, grid_h, grid_w):
    """Per-query decomposed rel-pos terms (unscaled query).

    [Candle PR 3280], Key Changes (term_h / term_w biases injected into the
    scores) and [mlx-examples issue 1451], body (SAM's add_decomposed_rel_pos):
        term_h[b,h,i,y] = sum_c q[b,h,i,c] * rel_pos_h[row(i) - y + grid_h - 1, c]
        term_w[b,h,i,x] = sum_c q[b,h,i,c] * rel_pos_w[col(i) - x + grid_w - 1, c]
    The gathered table for each query is built first, then one library
    contraction per term forms the dot products.
    Returns (term_h [B,H,T,grid_h], term_w [B,H,T,grid_w]) in float64.
    """
    q = np.asarray(q_bhsd, dtype=np.float64)
    rh = np.asarray(rel_pos_h, dtype=np.float64)
    rw = np.asarray(rel_pos_w, dtype=np.float64)
    T = q.shape[2]
    if T != grid_h * grid_w:
        raise ValueError("sequence length must equal grid_h * grid_w")
    if rh.shape != (2 * grid_h - 1, q.shape[3]) or rw.shape != (2 * grid_w - 1, q.shape[3]):
        raise ValueError("rel-pos tables must be [2*grid-1, head_dim]")
    t = np.arange(T)
    row, col = t // grid_w, t % grid_w
    gath_h = rh[_relpos_index(grid_h)[row]]      # [T, grid_h, D]
    gath_w = rw[_relpos_index(grid_w)[col]]      # [T, grid_w, D]
    term_h = np.einsum("bhid,iyd->bhiy", q, gath_h)
    term_w = np.einsum("bhid,ixd->bhix", q, gath_w)
    return term_h, term_w


def relpos_bias(term_h, term_w, grid_h, grid_w, rows=None):
    """bias[b,h,i,j] = term_h[b,h,i,row(j)] + term_w[b,h,i,col(j)].

    [Candle PR 3280], Key Changes: the term rows are broadcast over the key
    grid.  `rows` optionally restricts the query rows (for sampled checks).
    """
    th = np.asarray(term_h, dtype=np.float64)
    tw = np.asarray(term_w, dtype=np.float64)
    if rows is not None:
        th, tw = th[..., rows, :], tw[..., rows, :]
    j = np.arange(grid_h * grid_w)
    return th[..., j // grid_w] + tw[..., j % grid_w]


# ------------------------------------------------------------------ masks ---
def mask_bias(mask, Tq, Tkv, rows=None):
    """Additive bias (0 / -inf, or the caller's values) for one mask spec.

    [Axon PR 650], description (`:mask` options) and [mlx-examples issue 1451],
    body (an additive array broadcast to [B, N, T_q, T_kv]).  Index masks
    return [len(rows), Tkv]; tensor masks return the caller's array (rows
    selected on its query axis when it is not broadcast there).
    mask: None | {"kind": "causal", "offset": d}
               | {"kind": "sliding", "window": w, "offset": d}
               | {"kind": "additive", "data": M} | {"kind": "bool", "data": M}
    """
    if mask is None:
        return 0.0
    kind = mask["kind"]
    i = np.arange(Tq) if rows is None else np.asarray(rows)
    j = np.arange(Tkv)
    if kind in ("causal", "sliding"):
        d = int(mask.get("offset", 0))
        allowed = j[None, :] <= i[:, None] + d
        if kind == "sliding":
            w = int(mask["window"])
            if w < 1:
                raise ValueError("window must be >= 1")
            allowed &= j[None, :] > i[:, None] + d - w
        return np.where(allowed, 0.0, -np.inf)
    data = np.asarray(mask["data"])
    if data.ndim != 4:
        raise ValueError("tensor masks are rank-4, broadcastable to [B, Hq, Tq, Tkv]")
    if rows is not None and data.shape[2] != 1:
        data = data[:, :, rows, :]
    if kind == "additive":
        return data.astype(np.float64)
    if kind == "bool":
        return np.where(data.astype(bool), 0.0, -np.inf)
    raise ValueError(f"unknown mask kind {kind!r}")


# ---------------------------------------------------------------- softmax ---
def softmax_rows(z):
    """Row softmax over the last axis, plus the row log-sum-exp.

    [mlx-examples issue 1451], body: softmax(attn, axis=-1).  The row maximum
    is subtracted before exponentiating (exact up to rounding).  A row whose
    every entry is -inf has probabilities 0 and lse -inf.
    """
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    dead = np.isneginf(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(z - m_safe)
    s = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(dead, 0.0, e / np.where(dead, 1.0, s))
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, s)))
    return p, lse[..., 0]


# --------------------------------------------------------------- attention ---
def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be rank-4")
    B, Hq, Tq, D = q.shape
    if k.shape[0] != B or v.shape[0] != B or k.shape[3] != D or v.shape[3] != D:
        raise ValueError("batch / head_dim mismatch")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Tq, k.shape[2], D


def _prepare(q, k, v, layout, scale, rel_pos):
    q = to_bhsd(np.asarray(q, dtype=np.float64), layout)
    k = to_bhsd(np.asarray(k, dtype=np.float64), layout)
    v = to_bhsd(np.asarray(v, dtype=np.float64), layout)
    B, Hq, Hkv, Tq, Tkv, D = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)          # [Axon PR 650]: default 1/sqrt(head_dim)
    terms = None
    if rel_pos is not None:
        gh, gw = rel_pos["grid"]
        if Tq != gh * gw or Tkv != gh * gw:
            raise ValueError("rel-pos needs T_q = T_kv = grid_h * grid_w")
        terms = relpos_terms(q, rel_pos["rel_pos_h"], rel_pos["rel_pos_w"], gh, gw)
    return q, k, v, (B, Hq, Hkv, Tq, Tkv, D), float(scale), terms


def _bias_rows(b, h, rows, dims, mask, rel_pos, terms):
    """Bias for query rows `rows` of (b, h): [len(rows), Tkv] (or broadcastable)."""
    B, Hq, Hkv, Tq, Tkv, D = dims
    bias = np.zeros((len(rows), Tkv))
    if terms is not None:
        gh, gw = rel_pos["grid"]
        bias = bias + relpos_bias(terms[0][b, h], terms[1][b, h], gh, gw, rows=rows)
    mb = mask_bias(mask, Tq, Tkv, rows=rows)
    if isinstance(mb, np.ndarray) and mb.ndim == 4:
        mb = np.broadcast_to(mb, (mb.shape[0] if mb.shape[0] > 1 else B,
                                  mb.shape[1] if mb.shape[1] > 1 else Hq,
                                  len(rows) if mb.shape[2] > 1 else 1, Tkv))
        mb = mb[b if mb.shape[0] > 1 else 0, h if mb.shape[1] > 1 else 0]
    return bias + mb


def _attend(qr, kk, vv, bias, scale):
    """The definition for a block of query rows of one (batch, head):
    S = scale * q . K^T  ([Axon PR 650]: Q . K^T * scale), Z = S + bias,
    P = softmax_rows(Z), O = P . V  ([Axon PR 650] review diff: contraction
    of the weights with V over the key axis)."""
    s = scale * (qr @ kk.T)
    z = s + bias
    p, lse = softmax_rows(z)
    return p @ vv, lse, s, p


def sdpa(q, k, v, *, layout="bhsd", scale=None, mask=None, rel_pos=None,
         return_intermediates=False):
    """Full attention.  q [B,Hq,Tq,D], k/v [B,Hkv,Tkv,D] in `layout`.

    rel_pos: None | {"rel_pos_h": [2gh-1, D], "rel_pos_w": [2gw-1, D], "grid": (gh, gw)}
    Returns {"o": O in `layout` (float64), "lse": [B,Hq,Tq], and, when
    return_intermediates, "s", "bias", "p" as [B,Hq,Tq,Tkv] plus "terms"}.
    """
    q, k, v, dims, scale, terms = _prepare(q, k, v, layout, scale, rel_pos)
    B, Hq, Hkv, Tq, Tkv, D = dims
    o = np.zeros((B, Hq, Tq, D))
    lse = np.zeros((B, Hq, Tq))
    inter = {}
    if return_intermediates:
        inter = {"s": np.zeros((B, Hq, Tq, Tkv)), "bias": np.zeros((B, Hq, Tq, Tkv)),
                 "p": np.zeros((B, Hq, Tq, Tkv))}
    rows = np.arange(Tq)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            bias = _bias_rows(b, h, rows, dims, mask, rel_pos, terms)
            ob, lb, sb, pb = _attend(q[b, h], k[b, g], v[b, g], bias, scale)
            o[b, h], lse[b, h] = ob, lb
            if return_intermediates:
                inter["s"][b, h] = sb
                inter["bias"][b, h] = np.broadcast_to(bias, (Tq, Tkv))
                inter["p"][b, h] = pb
    out = {"o": from_bhsd(o, layout), "lse": lse}
    out.update(inter)
    if return_intermediates and terms is not None:
        out["terms"] = terms
    return out


def sdpa_rows(q, k, v, picks, *, layout="bhsd", scale=None, mask=None, rel_pos=None):
    """The same definition evaluated only at chosen output rows.

    picks: iterable of (b, h, i).  Each row of the definition depends only on
    its own query row, so a subset is exact.  Returns (o [n, D], lse [n]) in
    the order of `picks`.
    """
    q, k, v, dims, scale, terms = _prepare(q, k, v, layout, scale, None)
    B, Hq, Hkv, Tq, Tkv, D = dims
    picks = [tuple(int(x) for x in p) for p in picks]
    if rel_pos is not None:
        gh, gw = rel_pos["grid"]
        if Tq != gh * gw or Tkv != gh * gw:
            raise ValueError("rel-pos needs T_q = T_kv = grid_h * grid_w")
    groups = {}
    for n, (b, h, i) in enumerate(picks):
        groups.setdefault((b, h), []).append((n, i))
    o = np.zeros((len(picks), D))
    lse = np.zeros(len(picks))
    for (b, h), lst in groups.items():
        idx = np.array([n for n, _ in lst])
        rows = np.array([i for _, i in lst])
        g = kv_head_of(h, Hq, Hkv)
        terms = None
        if rel_pos is not None:
            th, tw = relpos_terms(q[b:b + 1, h:h + 1, :, :], rel_pos["rel_pos_h"],
                                  rel_pos["rel_pos_w"], gh, gw)
            terms = (np.zeros((B, Hq) + th.shape[2:]), np.zeros((B, Hq) + tw.shape[2:]))
            terms[0][b, h], terms[1][b, h] = th[0, 0], tw[0, 0]
        bias = _bias_rows(b, h, rows, dims, mask, rel_pos, terms)
        ob, lb, _, _ = _attend(q[b, h, rows], k[b, g], v[b, g], bias, scale)
        o[idx], lse[idx] = ob, lb
    return o, lse
