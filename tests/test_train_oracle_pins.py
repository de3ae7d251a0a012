"""Pins for the training-path oracle (dropout, attention weights, gradients).

Each check comes from something other than the oracle's own formulas:
published known-answer vectors of the generator, central finite differences
of the (separately pinned) forward definition, torch's CPU autograd in
float64 on the plain composition, closed forms and invariants.  The last
test plants slips in a copy of the gradient code and shows the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sdpa_oracle as so
from oracle import sdpa_train_oracle as st

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------ Philox --
def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        out = st.philox4x32_10([int(x, 16) for x in vec["ctr"]], [int(x, 16) for x in vec["key"]])
        assert ["%08x" % int(o) for o in out] == vec["out"]


def test_philox_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(1)
    ctr = rng.integers(0, 2**32, size=(4, 17), dtype=np.uint64)
    key = rng.integers(0, 2**32, size=(2,), dtype=np.uint64)
    vec = st.philox4x32_10(list(ctr), [int(key[0]), int(key[1])])
    for n in range(17):
        one = st.philox4x32_10([int(ctr[w, n]) for w in range(4)], [int(key[0]), int(key[1])])
        assert [int(x) for x in one] == [int(vec[w][n]) for w in range(4)]


def test_dropout_stream_mapping():
    """Element (b, h, i, j) reads half j % 8 of Philox((j // 8, i, b*Hq + h, step), seed)."""
    seed, step, rate = 0x123456789ABCDEF0, 7, 0.3
    B, Hq, Tq, Tkv = 2, 3, 5, 21
    keep = st.dropout_keep(seed, step, rate, B, Hq, Tq, Tkv)
    thresh, _ = st.dropout_threshold(rate)
    for (b, h, i, j) in [(0, 0, 0, 0), (1, 2, 4, 20), (0, 1, 3, 9), (1, 0, 2, 15), (1, 2, 0, 16)]:
        words = st.philox4x32_10([j // 8, i, b * Hq + h, step], [seed & 0xFFFFFFFF, seed >> 32])
        w = int(words[(j % 8) // 2])
        u = (w >> (16 * (j % 2))) & 0xFFFF
        assert keep[b, h, i, j] == (u >= thresh)


def test_dropout_rate_and_threshold():
    assert st.dropout_threshold(0.0) == (0, 1.0)
    t, s = st.dropout_threshold(0.1)
    assert t == 6554 and s == pytest.approx(65536.0 / (65536 - 6554))
    assert st.dropout_threshold(0.999999)[0] == 65535
    with pytest.raises(ValueError):
        st.dropout_threshold(1.0)
    keep = st.dropout_keep(42, 0, 0.0, 1, 2, 8, 40)
    assert keep.all()
    # kept fraction within 6 sigma of the binomial expectation
    rate = 0.25
    keep = st.dropout_keep(5, 3, rate, 2, 4, 64, 200)
    t, _ = st.dropout_threshold(rate)
    p = 1.0 - t / 65536.0
    n = keep.size
    assert abs(keep.mean() - p) < 6 * math.sqrt(p * (1 - p) / n)
    # different steps and seeds give different streams
    assert (st.dropout_keep(5, 4, rate, 2, 4, 64, 200) != keep).mean() > 0.2
    assert (st.dropout_keep(6, 3, rate, 2, 4, 64, 200) != keep).mean() > 0.2


def test_keep_words_round_trip():
    rng = np.random.default_rng(2)
    for Tkv in (1, 31, 32, 33, 100):
        keep = rng.random((2, 3, Tkv)) < 0.6
        words = st.pack_keep_words(keep)
        assert words.shape == (2, 3, (Tkv + 31) // 32) and words.dtype == np.uint32
        assert (st.unpack_keep_words(words, Tkv) == keep).all()
        # bit j % 32 of word j // 32, zero past the end
        j = Tkv - 1
        assert ((words[1, 2, j // 32] >> np.uint32(j % 32)) & 1) == keep[1, 2, j]
        if Tkv % 32:
            assert np.all(words[..., -1] >> np.uint32(Tkv % 32) == 0)


# -------------------------------------------------------- weights / forward --
def test_attention_weights_are_the_forward_softmax():
    rng = np.random.default_rng(3)
    q, k, v = rnd(rng, 1, 2, 7, 8), rnd(rng, 1, 2, 9, 8), rnd(rng, 1, 2, 9, 8)
    mask = {"kind": "causal", "offset": 1}
    w = st.attention_weights(q, k, mask=mask)
    ref = so.sdpa(q, k, v, mask=mask, return_intermediates=True)["p"]
    assert np.allclose(w, ref, atol=1e-14)
    assert np.allclose(w.sum(-1), 1.0)
    keep = rng.random(w.shape) < 0.7
    _, s = st.dropout_threshold(0.3)
    assert np.allclose(st.attention_weights(q, k, mask=mask, keep=keep, rate=0.3), ref * keep * s, atol=1e-14)


def test_train_forward_special_cases():
    rng = np.random.default_rng(4)
    q, k, v = rnd(rng, 1, 2, 6, 4), rnd(rng, 1, 2, 10, 4), rnd(rng, 1, 2, 10, 4)
    base = so.sdpa(q, k, v)
    allkeep = np.ones((1, 2, 6, 10), dtype=bool)
    out = st.sdpa_train_fwd(q, k, v, keep=allkeep, rate=0.0)
    assert np.allclose(out["o"], base["o"], atol=1e-13) and np.allclose(out["lse"], base["lse"])
    # one kept key per row: O_i = W_ij * Z * v_j
    jstar = rng.integers(0, 10, size=6)
    keep = np.zeros((1, 2, 6, 10), dtype=bool)
    keep[0, :, np.arange(6), jstar] = True
    rate = 0.5
    _, s = st.dropout_threshold(rate)
    W = so.sdpa(q, k, v, return_intermediates=True)["p"]
    o = st.sdpa_train_fwd(q, k, v, keep=keep, rate=rate)["o"]
    for h in range(2):
        for i in range(6):
            assert np.allclose(o[0, h, i], W[0, h, i, jstar[i]] * s * v[0, h, jstar[i]], atol=1e-13)
    # lse is the undropped one
    assert np.allclose(st.sdpa_train_fwd(q, k, v, keep=keep, rate=rate)["lse"], base["lse"])


def test_dropout_is_unbiased_on_average():
    rng = np.random.default_rng(5)
    q, k, v = rnd(rng, 1, 1, 4, 4), rnd(rng, 1, 1, 12, 4), rnd(rng, 1, 1, 12, 4)
    base = so.sdpa(q, k, v)["o"]
    rate, n = 0.4, 400
    acc = np.zeros_like(base)
    for s in range(n):
        keep = st.dropout_keep(1000 + s, 0, rate, 1, 1, 4, 12)
        acc += st.sdpa_train_fwd(q, k, v, keep=keep, rate=rate)["o"]
    # standard error of the mean is below ~0.05 for these magnitudes
    assert np.max(np.abs(acc / n - base)) < 0.08


# ------------------------------------------------------------- gradients --
def _loss(fwd, G):
    return float(np.sum(fwd * G))


def _fd_check(fn_o, args, grads, G, rng, npoints=6, eps=1e-6, rtol=1e-5):
    """Central differences of L = sum(O * G) at random coordinates of each argument."""
    for name, x in args.items():
        g = grads[name]
        for _ in range(npoints):
            idx = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            fd = (_loss(fn_o(**{**args, name: xp}), G) - _loss(fn_o(**{**args, name: xm}), G)) / (2 * eps)
            assert abs(fd - g[idx]) <= rtol * max(1.0, abs(fd)), (name, idx, fd, g[idx])


CASES = [
    dict(name="plain", Hq=2, Hkv=2, Tq=5, Tkv=7, mask=None, layout="bhsd"),
    dict(name="gqa_bshd", Hq=4, Hkv=2, Tq=6, Tkv=6, mask=None, layout="bshd"),
    dict(name="causal_offset", Hq=2, Hkv=1, Tq=6, Tkv=8, mask={"kind": "causal", "offset": 2}, layout="bhsd"),
    dict(name="sliding", Hq=2, Hkv=2, Tq=7, Tkv=7, mask={"kind": "sliding", "window": 3, "offset": 0},
         layout="bhsd"),
    dict(name="dead_rows", Hq=1, Hkv=1, Tq=6, Tkv=5, mask={"kind": "causal", "offset": -2}, layout="bhsd"),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
@pytest.mark.parametrize("drop", [False, True])
def test_backward_matches_finite_differences(case, drop):
    rng = np.random.default_rng(11)
    B, D = 2, 4
    Hq, Hkv, Tq, Tkv, lay = case["Hq"], case["Hkv"], case["Tq"], case["Tkv"], case["layout"]
    shp = (lambda H, T: (B, H, T, D)) if lay == "bhsd" else (lambda H, T: (B, T, H, D))
    q, k, v = rnd(rng, *shp(Hq, Tq)), rnd(rng, *shp(Hkv, Tkv)), rnd(rng, *shp(Hkv, Tkv))
    G = rnd(rng, *shp(Hq, Tq))
    keep, rate = (None, 0.0)
    if drop:
        rate = 0.3
        keep = st.dropout_keep(9, 1, rate, B, Hq, Tq, Tkv)
    kw = dict(layout=lay, scale=0.7, mask=case["mask"], keep=keep, rate=rate)
    grads = st.sdpa_bwd(q, k, v, G, **kw)
    fn = lambda q, k, v: st.sdpa_train_fwd(q, k, v, **kw)["o"]
    _fd_check(fn, {"q": q, "k": k, "v": v}, {"q": grads["dq"], "k": grads["dk"], "v": grads["dv"]}, G, rng)
    if case["name"] == "dead_rows":        # rows 0 and 1 see no key: zero gradient
        assert np.all(so.to_bhsd(grads["dq"], lay)[:, :, :2] == 0)


def test_backward_tensor_masks_finite_differences():
    rng = np.random.default_rng(12)
    B, H, Tq, Tkv, D = 1, 2, 5, 6, 4
    q, k, v = rnd(rng, B, H, Tq, D), rnd(rng, B, H, Tkv, D), rnd(rng, B, H, Tkv, D)
    G = rnd(rng, B, H, Tq, D)
    for mask in ({"kind": "additive", "data": rnd(rng, 1, H, Tq, Tkv)},
                 {"kind": "bool", "data": rng.random((B, 1, Tq, Tkv)) < 0.7}):
        grads = st.sdpa_bwd(q, k, v, G, mask=mask)
        fn = lambda q, k, v: st.sdpa_train_fwd(q, k, v, mask=mask)["o"]
        _fd_check(fn, {"q": q, "k": k, "v": v}, {"q": grads["dq"], "k": grads["dk"], "v": grads["dv"]}, G, rng)


def test_backward_relpos_finite_differences():
    rng = np.random.default_rng(13)
    B, H, gh, gw, D = 1, 2, 2, 3, 4
    T = gh * gw
    q, k, v = rnd(rng, B, H, T, D), rnd(rng, B, H, T, D), rnd(rng, B, H, T, D)
    rh, rw = rnd(rng, 2 * gh - 1, D), rnd(rng, 2 * gw - 1, D)
    G = rnd(rng, B, H, T, D)
    rp = lambda rh, rw: {"rel_pos_h": rh, "rel_pos_w": rw, "grid": (gh, gw)}
    grads = st.sdpa_bwd(q, k, v, G, rel_pos=rp(rh, rw))
    fn = lambda q, k, v, rh, rw: st.sdpa_train_fwd(q, k, v, rel_pos=rp(rh, rw))["o"]
    _fd_check(fn, {"q": q, "k": k, "v": v, "rh": rh, "rw": rw},
              {"q": grads["dq"], "k": grads["dk"], "v": grads["dv"], "rh": grads["drel_pos_h"],
               "rw": grads["drel_pos_w"]}, G, rng, npoints=8)



def test_backward_relpos_dropout_finite_differences():
    """Dropout together with the rel-pos bias: the gradients of q, k, v and of
    both tables against central differences of the dropped forward pass."""
    rng = np.random.default_rng(15)
    B, H, gh, gw, D = 1, 2, 3, 2, 4
    T = gh * gw
    q, k, v = rnd(rng, B, H, T, D), rnd(rng, B, H, T, D), rnd(rng, B, H, T, D)
    rh, rw = rnd(rng, 2 * gh - 1, D), rnd(rng, 2 * gw - 1, D)
    G = rnd(rng, B, H, T, D)
    rate = 0.3
    keep = st.dropout_keep(17, 2, rate, B, H, T, T)
    assert 0 < keep.mean() < 1
    rp = lambda rh, rw: {"rel_pos_h": rh, "rel_pos_w": rw, "grid": (gh, gw)}
    grads = st.sdpa_bwd(q, k, v, G, rel_pos=rp(rh, rw), keep=keep, rate=rate)
    fn = lambda q, k, v, rh, rw: st.sdpa_train_fwd(q, k, v, rel_pos=rp(rh, rw), keep=keep, rate=rate)["o"]
    _fd_check(fn, {"q": q, "k": k, "v": v, "rh": rh, "rw": rw},
              {"q": grads["dq"], "k": grads["dk"], "v": grads["dv"], "rh": grads["drel_pos_h"],
               "rw": grads["drel_pos_w"]}, G, rng, npoints=8)


def test_relpos_dropout_forward_keeps_one_key():
    """With one kept key j* per row, O_i = W[i, j*] * keep_scale * V[j*], where
    W[i, j*] = exp(scale q_i.k_j* + bias_ij* - lse_i) from the plain rel-pos
    oracle's lse: dropout and the bias compose as the pages state."""
    rng = np.random.default_rng(16)
    B, H, gh, gw, D = 1, 2, 2, 3, 4
    T = gh * gw
    q, k, v = rnd(rng, B, H, T, D), rnd(rng, B, H, T, D), rnd(rng, B, H, T, D)
    rh, rw = rnd(rng, 2 * gh - 1, D), rnd(rng, 2 * gw - 1, D)
    rp = {"rel_pos_h": rh, "rel_pos_w": rw, "grid": (gh, gw)}
    jstar = 4
    keep = np.zeros((B, H, T, T), dtype=bool)
    keep[..., jstar] = True
    rate = 0.25
    _, ks = st.dropout_threshold(rate)
    out = st.sdpa_train_fwd(q, k, v, scale=0.5, rel_pos=rp, keep=keep, rate=rate)
    base = so.sdpa(q, k, v, scale=0.5, rel_pos=rp)
    assert np.allclose(out["lse"], base["lse"], atol=1e-13)
    for h in range(H):
        for i in range(T):
            th = q[0, h, i] @ rh[i // gw - jstar // gw + gh - 1]      # term_h[i, row(j*)]
            tw = q[0, h, i] @ rw[i % gw - jstar % gw + gw - 1]        # term_w[i, col(j*)]
            w = np.exp(0.5 * q[0, h, i] @ k[0, h, jstar] + th + tw - base["lse"][0, h, i])
            assert np.allclose(out["o"][0, h, i], w * ks * v[0, h, jstar], atol=1e-12)

def test_backward_matches_torch_autograd():
    """torch's CPU autograd (float64) on the plain composition softmax -> dropout factor -> @ V."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, Tq, Tkv, D = 2, 4, 2, 9, 11, 8
    q, k, v = rnd(rng, B, Hq, Tq, D), rnd(rng, B, Hkv, Tkv, D), rnd(rng, B, Hkv, Tkv, D)
    G = rnd(rng, B, Hq, Tq, D)
    rate = 0.2
    keep = st.dropout_keep(3, 0, rate, B, Hq, Tq, Tkv)
    _, ks = st.dropout_threshold(rate)
    mask = {"kind": "sliding", "window": 4, "offset": 2}
    grads = st.sdpa_bwd(q, k, v, G, scale=0.5, mask=mask, keep=keep, rate=rate)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    rep = Hq // Hkv
    kk, vv = tk.repeat_interleave(rep, dim=1), tv.repeat_interleave(rep, dim=1)
    i = torch.arange(Tq)[:, None]
    j = torch.arange(Tkv)[None, :]
    allowed = (j <= i + 2) & (j > i + 2 - 4)
    z = 0.5 * tq @ kk.transpose(-1, -2)
    z = z.masked_fill(~allowed, float("-inf"))
    w = torch.softmax(z, dim=-1) * torch.tensor(np.where(keep, ks, 0.0))
    o = w @ vv
    (o * torch.tensor(G)).sum().backward()
    assert np.allclose(grads["dq"], tq.grad.numpy(), atol=1e-12)
    assert np.allclose(grads["dk"], tk.grad.numpy(), atol=1e-12)
    assert np.allclose(grads["dv"], tv.grad.numpy(), atol=1e-12)


def test_planted_gradient_slips_are_caught():
    """Slips in a copy of the gradient formula (sign of the row term, a missing
    dropout factor, the softmax Jacobian left out of dK, a wrong scale) fail the
    finite-difference pin."""
    rng = np.random.default_rng(15)
    B, H, Tq, Tkv, D = 1, 1, 4, 5, 3
    q, k, v = rnd(rng, B, H, Tq, D), rnd(rng, B, H, Tkv, D), rnd(rng, B, H, Tkv, D)
    G = rnd(rng, B, H, Tq, D)
    rate = 0.3
    keep = st.dropout_keep(1, 0, rate, B, H, Tq, Tkv)
    _, ks = st.dropout_threshold(rate)
    Z = np.where(keep, ks, 0.0)[0, 0]
    scale = 0.8

    def grads(slip):
        W = so.sdpa(q, k, v, scale=scale, return_intermediates=True)["p"][0, 0]
        dW = G[0, 0] @ v[0, 0].T
        if slip != "no_z":
            dW = dW * Z
        row = np.sum(W * dW, axis=1, keepdims=True)
        dZs = W * (dW + row) if slip == "sign" else W * (dW - row)
        dq = (1.0 if slip == "scale" else scale) * (dZs @ k[0, 0])
        dk = scale * ((dW.T @ q[0, 0]) if slip == "no_jacobian" else (dZs.T @ q[0, 0]))
        dv = (W * Z).T @ G[0, 0]
        return {"q": dq[None, None], "k": dk[None, None], "v": dv[None, None]}

    fn = lambda q, k, v: st.sdpa_train_fwd(q, k, v, scale=scale, keep=keep, rate=rate)["o"]
    _fd_check(fn, {"q": q, "k": k, "v": v}, grads(None), G, rng)
    for slip in ("sign", "no_z", "scale", "no_jacobian"):
        with pytest.raises(AssertionError):
            _fd_check(fn, {"q": q, "k": k, "v": v}, grads(slip), G, rng, npoints=12)
