"""Pins for the fp64 oracle: each check comes from something other than the
oracle itself -- a library routine (torch's CPU attention in float64), brute
force with pure-Python loops, closed forms, invariants of the definition, or
values derived by hand.  A plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a swapped h/w) fails one of them;
test_planted_mistakes_are_caught demonstrates that for several slips.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import sdpa_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def torch_ref(q, k, v, scale=None, attn_mask=None, is_causal=False, gqa=False):
    """torch's CPU attention in float64 on logical bhsd arrays."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).double()
    m = None
    if attn_mask is not None:
        m = torch.from_numpy(np.ascontiguousarray(attn_mask))
        m = m if m.dtype == torch.bool else m.double()
    out = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=is_causal,
                                         scale=scale, enable_gqa=gqa)
    return out.numpy()


# ------------------------------------------------------------ library routine
@pytest.mark.parametrize("scale", [None, 0.37])
def test_plain_matches_torch(scale):
    rng = np.random.default_rng(1)
    q, k, v = rnd(rng, 2, 3, 9, 5), rnd(rng, 2, 3, 11, 5), rnd(rng, 2, 3, 11, 5)
    got = oracle.sdpa(q, k, v, scale=scale)["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, scale=scale), atol=TOL, rtol=0)


def test_gqa_matches_torch_enable_gqa():
    rng = np.random.default_rng(2)
    q, k, v = rnd(rng, 2, 6, 7, 4), rnd(rng, 2, 2, 10, 4), rnd(rng, 2, 2, 10, 4)
    got = oracle.sdpa(q, k, v)["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, gqa=True), atol=TOL, rtol=0)
    # and equals MHA on repeat-interleaved K/V
    rep = oracle.sdpa(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1))["o"]
    np.testing.assert_allclose(got, rep, atol=TOL, rtol=0)


def test_causal_matches_torch_is_causal():
    rng = np.random.default_rng(3)
    q, k, v = rnd(rng, 1, 2, 13, 4), rnd(rng, 1, 2, 13, 4), rnd(rng, 1, 2, 13, 4)
    got = oracle.sdpa(q, k, v, mask={"kind": "causal", "offset": 0})["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, is_causal=True), atol=TOL, rtol=0)


@pytest.mark.parametrize("offset", [-3, 0, 4])
def test_causal_offset_matches_tril_mask(offset):
    rng = np.random.default_rng(4)
    Tq, Tkv = 9, 14
    q, k, v = rnd(rng, 1, 2, Tq, 3), rnd(rng, 1, 2, Tkv, 3), rnd(rng, 1, 2, Tkv, 3)
    allowed = torch.tril(torch.ones(Tq, Tkv, dtype=torch.bool), diagonal=offset).numpy()
    ref = torch_ref(q, k, v, attn_mask=allowed)
    got = oracle.sdpa(q, k, v, mask={"kind": "causal", "offset": offset})["o"]
    live = allowed.any(axis=1)
    np.testing.assert_allclose(got[:, :, live], ref[:, :, live], atol=TOL, rtol=0)
    assert np.all(got[:, :, ~live] == 0)


@pytest.mark.parametrize("w,offset", [(1, 0), (3, 0), (5, 2), (40, 0)])
def test_sliding_matches_band_mask(w, offset):
    rng = np.random.default_rng(5)
    T = 12
    q, k, v = rnd(rng, 1, 2, T, 3), rnd(rng, 1, 2, T, 3), rnd(rng, 1, 2, T, 3)
    ones = torch.ones(T, T, dtype=torch.bool)
    band = (torch.tril(ones, diagonal=offset) & ~torch.tril(ones, diagonal=offset - w)).numpy()
    got = oracle.sdpa(q, k, v, mask={"kind": "sliding", "window": w, "offset": offset})["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, attn_mask=band), atol=TOL, rtol=0)


@pytest.mark.parametrize("mshape", [(2, 3, 5, 8), (1, 1, 5, 8), (2, 1, 1, 8), (1, 3, 5, 1)])
def test_additive_mask_broadcast_matches_torch(mshape):
    rng = np.random.default_rng(6)
    q, k, v = rnd(rng, 2, 3, 5, 4), rnd(rng, 2, 3, 8, 4), rnd(rng, 2, 3, 8, 4)
    m = rnd(rng, *mshape)
    got = oracle.sdpa(q, k, v, mask={"kind": "additive", "data": m})["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, attn_mask=m), atol=TOL, rtol=0)


def test_bool_mask_matches_torch():
    rng = np.random.default_rng(7)
    q, k, v = rnd(rng, 2, 3, 6, 4), rnd(rng, 2, 3, 9, 4), rnd(rng, 2, 3, 9, 4)
    m = rng.random((2, 3, 6, 9)) < 0.6
    m[..., 0] = True     # keep every row alive for the library comparison
    got = oracle.sdpa(q, k, v, mask={"kind": "bool", "data": m})["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, attn_mask=m), atol=TOL, rtol=0)


def test_relpos_equals_additive_mask_route():
    """mlx-examples issue 1451, body: the rel-pos bias passed as an additive
    mask gives the same result as adding it to the materialised scores; here
    the bias is built by brute force and handed to torch as attn_mask."""
    rng = np.random.default_rng(8)
    gh, gw, D = 3, 4, 5
    T = gh * gw
    q, k, v = rnd(rng, 1, 2, T, D), rnd(rng, 1, 2, T, D), rnd(rng, 1, 2, T, D)
    rh, rw = rnd(rng, 2 * gh - 1, D), rnd(rng, 2 * gw - 1, D)
    bias = brute_relpos_bias(q, rh, rw, gh, gw)
    got = oracle.sdpa(q, k, v, rel_pos={"rel_pos_h": rh, "rel_pos_w": rw, "grid": (gh, gw)})["o"]
    np.testing.assert_allclose(got, torch_ref(q, k, v, attn_mask=bias), atol=TOL, rtol=0)


# ----------------------------------------------------------------- brute force
def brute_relpos_bias(q, rh, rw, gh, gw):
    """Pure-Python loops over the index formula term[q, k] = sum_c q[c] *
    table[q_coord - k_coord + grid - 1, c], bias = term_h[row] + term_w[col]."""
    B, H, T, D = q.shape
    out = np.zeros((B, H, T, T))
    for b in range(B):
        for h in range(H):
            for i in range(T):
                qh, qw = divmod(i, gw)
                for j in range(T):
                    kh, kw = divmod(j, gw)
                    th = math.fsum(q[b, h, i, c] * rh[qh - kh + gh - 1, c] for c in range(D))
                    tw = math.fsum(q[b, h, i, c] * rw[qw - kw + gw - 1, c] for c in range(D))
                    out[b, h, i, j] = th + tw
    return out


def brute_sdpa(q, k, v, scale, allowed, bias, kvmap):
    """Pure-Python loops: softmax over allowed keys of scale*q.k + bias, then P.V."""
    B, H, Tq, D = q.shape
    Tkv = k.shape[2]
    o = np.zeros((B, H, Tq, D))
    for b in range(B):
        for h in range(H):
            g = kvmap(h)
            for i in range(Tq):
                z = {}
                for j in range(Tkv):
                    if allowed(b, h, i, j):
                        z[j] = scale * math.fsum(q[b, h, i, c] * k[b, g, j, c] for c in range(D)) + bias(b, h, i, j)
                if not z:
                    continue
                m = max(z.values())
                e = {j: math.exp(x - m) for j, x in z.items()}
                s = math.fsum(e.values())
                for c in range(D):
                    o[b, h, i, c] = math.fsum(e[j] / s * v[b, g, j, c] for j in e)
    return o


@pytest.mark.parametrize("case", ["plain", "relpos", "causal", "sliding", "gqa", "additive", "bool"])
def test_brute_force(case):
    rng = np.random.default_rng(10)
    B, Hq, Hkv, D = 1, 2, 2, 3
    Tq = Tkv = 6
    kw = {}
    allowed = lambda b, h, i, j: True
    bias = lambda b, h, i, j: 0.0
    kvmap = lambda h: h
    if case == "gqa":
        Hq, Hkv = 4, 2
        kvmap = lambda h: h // 2
    if case == "additive":
        Tkv = 8
    q, k, v = rnd(rng, B, Hq, Tq, D), rnd(rng, B, Hkv, Tkv, D), rnd(rng, B, Hkv, Tkv, D)
    scale = 0.61
    if case == "relpos":
        gh, gw = 2, 3
        rh, rw = rnd(rng, 3, D), rnd(rng, 5, D)
        bm = brute_relpos_bias(q, rh, rw, gh, gw)
        bias = lambda b, h, i, j: bm[b, h, i, j]
        kw["rel_pos"] = {"rel_pos_h": rh, "rel_pos_w": rw, "grid": (gh, gw)}
    elif case == "causal":
        allowed = lambda b, h, i, j: j <= i + 1
        kw["mask"] = {"kind": "causal", "offset": 1}
    elif case == "sliding":
        allowed = lambda b, h, i, j: i - 2 < j <= i
        kw["mask"] = {"kind": "sliding", "window": 2, "offset": 0}
    elif case == "additive":
        m = rnd(rng, 1, Hq, 1, Tkv)
        bias = lambda b, h, i, j: m[0, h, 0, j]
        kw["mask"] = {"kind": "additive", "data": m}
    elif case == "bool":
        m = rng.random((B, Hq, Tq, Tkv)) < 0.5
        m[0, 0, 2, :] = False      # one fully masked row
        allowed = lambda b, h, i, j: bool(m[b, h, i, j])
        kw["mask"] = {"kind": "bool", "data": m}
    ref = brute_sdpa(q, k, v, scale, allowed, bias, kvmap)
    got = oracle.sdpa(q, k, v, scale=scale, **kw)["o"]
    np.testing.assert_allclose(got, ref, atol=TOL, rtol=0)


# -------------------------------------------------------------- rel-pos pins
def test_relpos_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "relpos_hand_2x3.json")))
    gh, gw = g["grid"]
    q = np.array(g["q"], dtype=float).reshape(1, 1, gh * gw, 1)
    rh = np.array(g["rel_pos_h"], dtype=float).reshape(-1, 1)
    rw = np.array(g["rel_pos_w"], dtype=float).reshape(-1, 1)
    th, tw = oracle.relpos_terms(q, rh, rw, gh, gw)
    bias = oracle.relpos_bias(th, tw, gh, gw)
    for tok, exp in g["term_h"].items():
        assert th[0, 0, int(tok)].tolist() == exp
    for tok, exp in g["term_w"].items():
        assert tw[0, 0, int(tok)].tolist() == exp
    for tok, exp in g["bias"].items():
        assert bias[0, 0, int(tok)].tolist() == exp


def test_relpos_terms_second_formulation():
    """Multiply first (A = Q . R^T over all 2g-1 offsets), gather afterwards:
    term[i, y] = A[i, coord(i) - y + g - 1] must equal gather-then-multiply."""
    rng = np.random.default_rng(11)
    gh, gw, D = 4, 5, 6
    T = gh * gw
    q = rnd(rng, 2, 3, T, D)
    rh, rw = rnd(rng, 2 * gh - 1, D), rnd(rng, 2 * gw - 1, D)
    th, tw = oracle.relpos_terms(q, rh, rw, gh, gw)
    Ah, Aw = q @ rh.T, q @ rw.T
    for i in range(T):
        r, c = divmod(i, gw)
        for y in range(gh):
            np.testing.assert_allclose(th[:, :, i, y], Ah[:, :, i, r - y + gh - 1], atol=TOL, rtol=0)
        for x in range(gw):
            np.testing.assert_allclose(tw[:, :, i, x], Aw[:, :, i, c - x + gw - 1], atol=TOL, rtol=0)


def test_relpos_zero_tables_is_plain_sdpa():
    rng = np.random.default_rng(12)
    q, k, v = rnd(rng, 1, 2, 12, 4), rnd(rng, 1, 2, 12, 4), rnd(rng, 1, 2, 12, 4)
    z = {"rel_pos_h": np.zeros((5, 4)), "rel_pos_w": np.zeros((7, 4)), "grid": (3, 4)}
    np.testing.assert_allclose(oracle.sdpa(q, k, v, rel_pos=z)["o"], torch_ref(q, k, v), atol=TOL, rtol=0)


def test_relpos_per_query_constant_in_term_h_leaves_output():
    """Adding c_i to every term_h[i, :] shifts row i of the bias by c_i, which
    softmax ignores.  A constant embedding e added to all rel_pos_h rows adds
    q_i . e to every term_h[i, y]; the output must not move (lse moves by it)."""
    rng = np.random.default_rng(13)
    gh, gw, D = 3, 3, 4
    q, k, v = rnd(rng, 1, 2, 9, D), rnd(rng, 1, 2, 9, D), rnd(rng, 1, 2, 9, D)
    rh, rw = rnd(rng, 5, D), rnd(rng, 5, D)
    e = rnd(rng, D)
    a = oracle.sdpa(q, k, v, rel_pos={"rel_pos_h": rh, "rel_pos_w": rw, "grid": (gh, gw)})
    b = oracle.sdpa(q, k, v, rel_pos={"rel_pos_h": rh + e, "rel_pos_w": rw, "grid": (gh, gw)})
    np.testing.assert_allclose(a["o"], b["o"], atol=1e-12, rtol=0)
    np.testing.assert_allclose(b["lse"] - a["lse"], q @ e, atol=1e-12, rtol=0)
    # but a term that varies with the key row does move it
    rh2 = rh.copy()
    rh2[gh - 1] += e
    c = oracle.sdpa(q, k, v, rel_pos={"rel_pos_h": rh2, "rel_pos_w": rw, "grid": (gh, gw)})
    assert np.abs(c["o"] - a["o"]).max() > 1e-3


def test_relpos_bias_depends_on_key_only_through_grid_coords():
    rng = np.random.default_rng(14)
    gh, gw = 3, 4
    th, tw = rnd(rng, 1, 1, 12, gh), rnd(rng, 1, 1, 12, gw)
    bias = oracle.relpos_bias(th, tw, gh, gw)
    for j in range(12):
        r, c = divmod(j, gw)
        np.testing.assert_allclose(bias[..., j], th[..., r] + tw[..., c], atol=0, rtol=0)


# --------------------------------------------------------------- closed forms
def test_single_key_gives_v():
    rng = np.random.default_rng(15)
    q, k, v = rnd(rng, 2, 2, 5, 3), rnd(rng, 2, 2, 1, 3), rnd(rng, 2, 2, 1, 3)
    o = oracle.sdpa(q, k, v)["o"]
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-15, rtol=0)


def test_equal_scores_give_mean_of_v_and_log_n_lse():
    rng = np.random.default_rng(16)
    T = 7
    q = np.zeros((1, 1, 4, 3))
    k, v = rnd(rng, 1, 1, T, 3), rnd(rng, 1, 1, T, 3)
    r = oracle.sdpa(q, k, v)
    np.testing.assert_allclose(r["o"][0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (4, 3)), atol=1e-14)
    np.testing.assert_allclose(r["lse"], math.log(T), atol=1e-14)
    # identical keys, random query: same
    k2 = np.broadcast_to(k[:, :, :1], k.shape)
    r2 = oracle.sdpa(rnd(rng, 1, 1, 4, 3), k2, v)
    np.testing.assert_allclose(r2["o"][0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (4, 3)), atol=1e-14)


def test_two_keys_logistic_closed_form():
    """Two keys: O = sigma(d) v0 + (1 - sigma(d)) v1 with
    d = scale q.(k0 - k1) + (bias0 - bias1), sigma the logistic function."""
    q = np.array([0.3, -1.2, 0.5]).reshape(1, 1, 1, 3)
    k = np.array([[1.0, 0.5, -0.25], [-0.5, 2.0, 1.0]]).reshape(1, 1, 2, 3)
    v = np.array([[2.0, -1.0, 0.0], [0.5, 3.0, -2.0]]).reshape(1, 1, 2, 3)
    bias = np.array([0.7, -0.4]).reshape(1, 1, 1, 2)
    scale = 0.8
    d = scale * float(q[0, 0, 0] @ (k[0, 0, 0] - k[0, 0, 1])) + (0.7 + 0.4)
    sig = 1.0 / (1.0 + math.exp(-d))
    expect = sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1]
    got = oracle.sdpa(q, k, v, scale=scale, mask={"kind": "additive", "data": bias})["o"][0, 0, 0]
    np.testing.assert_allclose(got, expect, atol=1e-15, rtol=0)


def test_probability_rows_sum_to_one():
    rng = np.random.default_rng(17)
    q, k, v = rnd(rng, 1, 2, 9, 4), rnd(rng, 1, 2, 9, 4), rnd(rng, 1, 2, 9, 4)
    r = oracle.sdpa(q, k, v, mask={"kind": "sliding", "window": 3, "offset": 0}, return_intermediates=True)
    np.testing.assert_allclose(r["p"].sum(axis=-1), 1.0, atol=1e-14)
    assert np.all(r["p"] >= 0)


def test_first_causal_row_is_v0_and_window_one_is_identity():
    rng = np.random.default_rng(18)
    q, k, v = rnd(rng, 2, 2, 8, 4), rnd(rng, 2, 2, 8, 4), rnd(rng, 2, 2, 8, 4)
    o = oracle.sdpa(q, k, v, mask={"kind": "causal", "offset": 0})["o"]
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-15, rtol=0)
    o1 = oracle.sdpa(q, k, v, mask={"kind": "sliding", "window": 1, "offset": 0})["o"]
    np.testing.assert_allclose(o1, v, atol=1e-15, rtol=0)
    big = oracle.sdpa(q, k, v, mask={"kind": "sliding", "window": 8, "offset": 0})["o"]
    np.testing.assert_allclose(big, o, atol=0, rtol=0)


def test_allowed_key_count_of_sliding_window():
    rng = np.random.default_rng(19)
    T, w = 10, 4
    q, k, v = rnd(rng, 1, 1, T, 2), rnd(rng, 1, 1, T, 2), rnd(rng, 1, 1, T, 2)
    p = oracle.sdpa(q, k, v, mask={"kind": "sliding", "window": w, "offset": 0}, return_intermediates=True)["p"]
    assert [(p[0, 0, i] > 0).sum() for i in range(T)] == [min(i + 1, w) for i in range(T)]


def test_fully_masked_row_is_zero_with_neg_inf_lse():
    rng = np.random.default_rng(20)
    q, k, v = rnd(rng, 1, 1, 3, 2), rnd(rng, 1, 1, 4, 2), rnd(rng, 1, 1, 4, 2)
    m = np.ones((1, 1, 3, 4), dtype=bool)
    m[0, 0, 1] = False
    r = oracle.sdpa(q, k, v, mask={"kind": "bool", "data": m})
    assert np.all(r["o"][0, 0, 1] == 0) and np.isneginf(r["lse"][0, 0, 1])
    assert np.all(np.isfinite(r["o"]))
    r2 = oracle.sdpa(q, k, v, mask={"kind": "causal", "offset": -10})
    assert np.all(r2["o"] == 0) and np.all(np.isneginf(r2["lse"]))


def test_lse_matches_logsumexp():
    rng = np.random.default_rng(21)
    q, k, v = rnd(rng, 1, 2, 5, 3), rnd(rng, 1, 2, 6, 3), rnd(rng, 1, 2, 6, 3)
    r = oracle.sdpa(q, k, v, scale=0.9)
    s = 0.9 * np.einsum("bhid,bhjd->bhij", q, k)
    expect = torch.logsumexp(torch.from_numpy(s), dim=-1).numpy()
    np.testing.assert_allclose(r["lse"], expect, atol=1e-13, rtol=0)


def test_layouts_agree():
    rng = np.random.default_rng(22)
    q, k, v = rnd(rng, 2, 4, 6, 3), rnd(rng, 2, 2, 6, 3), rnd(rng, 2, 2, 6, 3)
    a = oracle.sdpa(q, k, v, mask={"kind": "causal"})["o"]
    t = lambda x: x.transpose(0, 2, 1, 3)
    b = oracle.sdpa(t(q), t(k), t(v), layout="bshd", mask={"kind": "causal"})["o"]
    np.testing.assert_array_equal(t(b), a)


def test_sampled_rows_equal_full():
    rng = np.random.default_rng(23)
    gh, gw = 3, 4
    q, k, v = rnd(rng, 2, 4, 12, 3), rnd(rng, 2, 2, 12, 3), rnd(rng, 2, 2, 12, 3)
    rp = {"rel_pos_h": rnd(rng, 5, 3), "rel_pos_w": rnd(rng, 7, 3), "grid": (gh, gw)}
    full = oracle.sdpa(q, k, v, rel_pos=rp)
    picks = [(0, 0, 0), (1, 3, 11), (0, 2, 5), (1, 1, 7)]
    o, lse = oracle.sdpa_rows(q, k, v, picks, rel_pos=rp)
    for n, (b, h, i) in enumerate(picks):
        np.testing.assert_allclose(o[n], full["o"][b, h, i], atol=1e-14)
        np.testing.assert_allclose(lse[n], full["lse"][b, h, i], atol=1e-14)
    m = {"kind": "sliding", "window": 3, "offset": 1}
    full = oracle.sdpa(q, k, v, layout="bshd", mask=m)
    o, _ = oracle.sdpa_rows(q, k, v, [(1, 2, 3), (0, 11, 1)], layout="bshd", mask=m)
    np.testing.assert_allclose(o[0], full["o"][1, 3, 2], atol=1e-14)   # bshd: [b, t, h, d]
    np.testing.assert_allclose(o[1], full["o"][0, 1, 11], atol=1e-14)


# ------------------------------------------------------------ planted slips
def test_planted_mistakes_are_caught(monkeypatch):
    """Plant plausible slips into the oracle (on the CPU) and check that the
    pins above notice each one."""
    g = json.load(open(os.path.join(GOLDEN, "relpos_hand_2x3.json")))
    gh, gw = g["grid"]
    q = np.array(g["q"], dtype=float).reshape(1, 1, gh * gw, 1)
    rh = np.array(g["rel_pos_h"], dtype=float).reshape(-1, 1)
    rw = np.array(g["rel_pos_w"], dtype=float).reshape(-1, 1)
    expect = np.array([g["bias"][str(t)] for t in (0, 4, 5)], dtype=float)

    def hand_bias():
        th, tw = so.relpos_terms(q, rh, rw, gh, gw)
        return so.relpos_bias(th, tw, gh, gw)[0, 0, [0, 4, 5]]

    assert np.array_equal(hand_bias(), expect)
    # 1) sign of the relative offset flipped
    monkeypatch.setattr(so, "_relpos_index", lambda n: (lambda c: c[None, :] - c[:, None] + n - 1)(np.arange(n)))
    assert not np.array_equal(hand_bias(), expect)
    monkeypatch.undo()
    # 2) key tokens read column-major on the grid (row = j % gh, col = j // gh)
    def colmajor(th, tw, a, b, rows=None):
        th, tw = np.asarray(th, float), np.asarray(tw, float)
        j = np.arange(a * b)
        return th[..., j % a] + tw[..., j // a]
    monkeypatch.setattr(so, "relpos_bias", colmajor)
    assert not np.array_equal(hand_bias(), expect)
    monkeypatch.undo()
    # 3) scale dropped from the scores: the closed two-key form catches it
    orig_attend = so._attend
    monkeypatch.setattr(so, "_attend", lambda qr, kk, vv, bias, scale: orig_attend(qr, kk, vv, bias, 1.0))
    with pytest.raises(AssertionError):
        test_two_keys_logistic_closed_form()
    monkeypatch.undo()
    # 4) K used untransposed-equivalent slip: V in place of K
    monkeypatch.setattr(so, "_attend", lambda qr, kk, vv, bias, scale: orig_attend(qr, vv, vv, bias, scale))
    with pytest.raises(AssertionError):
        test_plain_matches_torch(None)
    monkeypatch.undo()
    # 5) GQA mapping h % Hkv instead of h // (Hq // Hkv)
    monkeypatch.setattr(so, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        test_gqa_matches_torch_enable_gqa()
    monkeypatch.undo()
    # 6) sliding window one key too wide
    orig_mask = so.mask_bias

    def wide(mask, Tq, Tkv, rows=None):
        if mask and mask.get("kind") == "sliding":
            mask = dict(mask, window=mask["window"] + 1)
        return orig_mask(mask, Tq, Tkv, rows)
    monkeypatch.setattr(so, "mask_bias", wide)
    with pytest.raises(AssertionError):
        test_sliding_matches_band_mask(3, 0)
    monkeypatch.undo()
