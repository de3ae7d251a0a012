"""GPU parity of the training path (dropout keep bits, dropout forward,
attention weights, backward) against the fp64 oracle, through the C ABI.

Every oracle input comes from the seeded generators or from the oracle
itself (the keep bits the kernels consume are the oracle's Philox bits, the
forward output and lse handed to the backward kernels are the oracle's);
the GPU generator is checked separately, bit for bit.

Gradient tolerance (normalised error max|g_gpu - g| / max|g|): the kernels
round the weights and dS to the input type before the matrix products
(2^-9 relative for bf16, 2^-11 for fp16), take O in the input type for
rowsum(dO * O), and store the gradients in the input type.  Emulating
exactly those roundings in fp64 numpy on unit-normal inputs (T 333..1024,
head_dim 64 / 128) gives 3-5e-3 (bf16) and 4-7e-4 (fp16); the bounds below
are 3x that.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_train_oracle as st
from parity_util import TOL, max_err, np64

pytestmark = pytest.mark.gpu

GTOL = {torch.bfloat16: 1.5e-2, torch.float16: 2e-3}
DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def draw(rng, shape, dt):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(dt)


def shp(layout, B, H, T, D):
    return (B, H, T, D) if layout == "bhsd" else (B, T, H, D)


def keep_words_tensor(keep_bool):
    w = st.pack_keep_words(keep_bool)                      # uint32
    return torch.from_numpy(w.view(np.int32)).cuda()


def norm_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.all(np.isfinite(a))
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


# --------------------------------------------------------- dropout keep bits --
@pytest.mark.parametrize("seed,step,rate,shape", [
    (0, 0, 0.1, (1, 2, 5, 40)), (0x123456789ABCDEF0, 7, 0.3, (2, 3, 17, 97)),
    (42, 123456, 0.5, (1, 1, 64, 256)), (7, 1, 0.0, (1, 2, 3, 33)), (9, 2, 0.95, (2, 1, 9, 8)),
])
def test_dropout_mask_bits_match_oracle(gpu, seed, step, rate, shape):
    B, Hq, Tq, Tkv = shape
    got = gpu.dropout_mask(seed, step, rate, B, Hq, Tq, Tkv)
    torch.cuda.synchronize()
    ref = st.pack_keep_words(st.dropout_keep(seed, step, rate, B, Hq, Tq, Tkv))
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref)


def test_dropout_mask_large_rows(gpu):
    """A bench-sized score array (1 x 12 x 4096 x 4096), checked on sampled rows:
    the oracle's generator draws just those rows (counters depend only on
    (j // 8, i, b * Hq + h, step))."""
    B, Hq, Tq, Tkv, seed, step, rate = 1, 12, 4096, 4096, 5, 3, 0.1
    got = gpu.dropout_mask(seed, step, rate, B, Hq, Tq, Tkv).cpu().numpy().view(np.uint32)
    thresh, _ = st.dropout_threshold(rate)
    ng = Tkv // 8
    for (b, h, i) in [(0, 0, 0), (0, 11, 4095), (0, 5, 2049), (0, 7, 31)]:
        words = st.philox4x32_10((np.arange(ng), np.full(ng, i), np.full(ng, b * Hq + h), np.full(ng, step)),
                                 (seed, 0))
        halves = np.stack([x for w in words for x in (w & np.uint64(0xFFFF), w >> np.uint64(16))], axis=-1)
        row = st.pack_keep_words(halves.reshape(-1) >= np.uint64(thresh))
        assert np.array_equal(got[b, h, i], row)


# ------------------------------------------------------------ dropout forward --
FWD_CASES = [
    ("bf16", "bhsd", 2, 4, 2, 200, 333, 64, None),                       # matrix-core kernel, GQA
    ("bf16", "bshd", 1, 2, 2, 97, 130, 128, {"kind": "causal", "offset": 3}),
    ("bf16", "bhsd", 1, 2, 1, 150, 150, 64, {"kind": "sliding", "window": 40, "offset": 0}),
    ("bf16", "bhsd", 1, 2, 2, 70, 90, 64, "additive"),
    ("fp16", "bhsd", 1, 2, 2, 100, 77, 64, None),                        # generic kernel
    ("fp32", "bshd", 2, 2, 1, 65, 40, 48, {"kind": "causal", "offset": 0}),
    ("bf16", "bhsd", 1, 1, 1, 33, 50, 32, "bool"),
]


@pytest.mark.parametrize("tiled", [1, 0], ids=["tiled-on", "tiled-off"])
@pytest.mark.parametrize("case", FWD_CASES, ids=[f"{c[0]}-{c[1]}-D{c[7]}-{c[8] if isinstance(c[8], str) else (c[8] or {}).get('kind', 'none')}" for c in FWD_CASES])
def test_dropout_forward_matches_oracle(gpu, case, tiled):
    """Each case with the double-buffered kernel allowed (it takes 16-bit
    inputs at head_dim 64 / 128 with no mask or a causal / sliding mask) and
    with it switched off (the general MFMA kernel, else the generic one)."""
    dts, layout, B, Hq, Hkv, Tq, Tkv, D, mask = case
    dt = DT[dts]
    rng = np.random.default_rng(31)
    q = draw(rng, shp(layout, B, Hq, Tq, D), dt)
    k = draw(rng, shp(layout, B, Hkv, Tkv, D), dt)
    v = draw(rng, shp(layout, B, Hkv, Tkv, D), dt)
    omask = gmask = mask
    if mask == "additive":
        m = torch.from_numpy(rng.standard_normal((1, Hq, Tq, Tkv), dtype=np.float32))
        omask, gmask = {"kind": "additive", "data": m.numpy()}, {"kind": "additive", "data": m.cuda()}
    elif mask == "bool":
        m = torch.from_numpy(rng.random((B, 1, Tq, Tkv)) < 0.8)
        m[..., 0] = True
        omask, gmask = {"kind": "bool", "data": m.numpy()}, {"kind": "bool", "data": m.cuda()}
    rate = 0.2
    keep = st.dropout_keep(11, 4, rate, B, Hq, Tq, Tkv)
    scale = 1.0 / np.sqrt(D)
    gpu.set_tuning("tiled", tiled)
    try:
        o, lse = gpu.sdpa(q.cuda(), k.cuda(), v.cuda(), layout=layout, scale=scale, mask=gmask,
                          out_dtype=torch.float32, return_lse=True,
                          dropout={"keep": keep_words_tensor(keep), "rate": rate})
        torch.cuda.synchronize()
        kernel = gpu.last_kernel()
    finally:
        gpu.set_tuning("tiled", 1)
    eligible = dts != "fp32" and D in (64, 128) and (mask is None or isinstance(mask, dict))
    assert (kernel == "flash_tiled_kernel") == bool(tiled and eligible), kernel
    ref = st.sdpa_train_fwd(np64(q), np64(k), np64(v), layout=layout, scale=scale, mask=omask, keep=keep, rate=rate)
    # The forward tolerance of the same kernels, scaled by the kept weights' factor: the
    # weights carry the same rounding as without dropout and are multiplied by
    # 65536 / (65536 - thresh) = 1.25 at rate 0.2, so the error of O scales by that factor.
    assert max_err(np64(o), ref["o"]) < TOL[dts] * (65536.0 / (65536.0 - round(rate * 65536)))
    # lse comes from the row sum of the weights as rounded for P.V, like the forward pass without dropout
    assert max_err(np64(lse), ref["lse"]) <= TOL[dts]


# --------------------------------------------------------- attention weights --
WEIGHT_CASES = [
    # dtype, layout, B, Hq, Hkv, Tq, Tkv, D, mask, drop, matrix-core kernel
    ("bf16", "bhsd", 2, 2, 1, 70, 100, 64, None, False, True),
    ("bf16", "bhsd", 2, 2, 1, 70, 100, 64, {"kind": "causal", "offset": 1}, True, True),
    ("fp32", "bhsd", 2, 2, 1, 70, 100, 64, {"kind": "sliding", "window": 9, "offset": 0}, False, False),
    ("fp16", "bhsd", 2, 2, 1, 70, 100, 64, None, True, True),
    # 3 query blocks of 128 and 3 key ranges of 256, both ragged; GQA; bshd
    ("bf16", "bshd", 1, 4, 2, 300, 520, 128, {"kind": "sliding", "window": 100, "offset": 3}, True, True),
    ("bf16", "bhsd", 1, 2, 2, 130, 100, 32, {"kind": "causal", "offset": -40}, False, True),     # dead rows
    ("fp16", "bhsd", 1, 2, 1, 50, 90, 64, "additive", False, True),
    ("bf16", "bhsd", 1, 2, 2, 40, 70, 64, "bool", True, True),
    ("bf16", "bhsd", 1, 2, 2, 40, 70, 16, None, False, False),                                 # vector ALUs
]


@pytest.mark.parametrize("case", WEIGHT_CASES, ids=[
    f"{c[0]}-{c[1]}-{c[5]}x{c[6]}-D{c[7]}-{c[8] if isinstance(c[8], str) else (c[8] or {}).get('kind', 'none')}"
    f"{'-drop' if c[9] else ''}" for c in WEIGHT_CASES])
def test_attention_weights_match_oracle(gpu, case):
    """Weights against the oracle's, on the matrix-core kernel (16-bit inputs at head_dim 32 / 64 / 128)
    and on the vector-ALU kernel (fp32 inputs, other head dims), asserting which one ran."""
    dts, layout, B, Hq, Hkv, Tq, Tkv, D, mask, drop, mfma = case
    dt = DT[dts]
    rng = np.random.default_rng(32)
    q, k = draw(rng, shp(layout, B, Hq, Tq, D), dt), draw(rng, shp(layout, B, Hkv, Tkv, D), dt)
    v = draw(rng, shp(layout, B, Hkv, Tkv, D), dt)
    scale = 0.125
    omask = gmask = mask
    if mask == "additive":
        m = torch.from_numpy(rng.standard_normal((1, Hq, Tq, Tkv), dtype=np.float32))
        omask, gmask = {"kind": "additive", "data": m.numpy()}, {"kind": "additive", "data": m.cuda()}
    elif mask == "bool":
        m = torch.from_numpy(rng.random((B, 1, Tq, Tkv)) < 0.7)
        m[..., 0] = True
        omask, gmask = {"kind": "bool", "data": m.numpy()}, {"kind": "bool", "data": m.cuda()}
    keep, rate, dro = None, 0.0, None
    if drop:
        rate = 0.25
        keep = st.dropout_keep(3, 9, rate, B, Hq, Tq, Tkv)
        dro = {"keep": keep_words_tensor(keep), "rate": rate}
    lse = oracle.sdpa(np64(q), np64(k), np64(v), layout=layout, scale=scale, mask=omask)["lse"]
    w = gpu.attention_weights(q.cuda(), k.cuda(), torch.from_numpy(lse.astype(np.float32)).cuda(), layout=layout,
                              scale=scale, mask=gmask, dropout=dro)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == ("attn_weights_mfma_kernel" if mfma else "attn_weights_kernel")
    ref = st.attention_weights(np64(q), np64(k), layout=layout, scale=scale, mask=omask, keep=keep, rate=rate)
    assert max_err(np64(w), ref) < 2e-5


# ------------------------------------------------------------------ backward --
BWD_CASES = [
    # dtype, layout, B, Hq, Hkv, Tq, Tkv, D, mask, drop, grad fp32
    ("bf16", "bhsd", 1, 2, 2, 200, 333, 64, None, False, False),
    ("bf16", "bshd", 2, 4, 2, 97, 130, 128, None, False, False),
    ("bf16", "bhsd", 1, 8, 2, 333, 333, 128, {"kind": "causal", "offset": 0}, False, False),
    ("bf16", "bhsd", 1, 2, 2, 150, 150, 64, {"kind": "sliding", "window": 40, "offset": 0}, False, True),
    ("bf16", "bhsd", 1, 2, 2, 130, 100, 64, {"kind": "causal", "offset": -40}, False, False),   # dead rows
    ("bf16", "bhsd", 1, 2, 1, 96, 200, 32, "additive", False, False),
    ("bf16", "bshd", 1, 2, 2, 64, 64, 64, "bool", True, False),
    ("bf16", "bhsd", 2, 2, 2, 160, 224, 64, None, True, False),
    ("bf16", "bhsd", 1, 4, 1, 129, 257, 128, {"kind": "causal", "offset": 5}, True, True),
    ("fp16", "bhsd", 1, 2, 2, 200, 333, 64, None, False, False),
    ("fp16", "bshd", 1, 4, 2, 100, 77, 128, {"kind": "sliding", "window": 30, "offset": 2}, True, False),
    ("fp16", "bhsd", 1, 2, 2, 1, 5, 32, None, False, True),                                    # tiny
]


def _bwd_case_id(c):
    m = c[8] if isinstance(c[8], str) else (c[8] or {}).get("kind", "none")
    return f"{c[0]}-{c[1]}-{c[3]}x{c[4]}-{c[5]}x{c[6]}-D{c[7]}-{m}{'-drop' if c[9] else ''}{'-g32' if c[10] else ''}"


@pytest.mark.parametrize("case", BWD_CASES, ids=[_bwd_case_id(c) for c in BWD_CASES])
def test_backward_matches_oracle(gpu, case):
    dts, layout, B, Hq, Hkv, Tq, Tkv, D, mask, drop, g32 = case
    dt = DT[dts]
    rng = np.random.default_rng(33)
    q = draw(rng, shp(layout, B, Hq, Tq, D), dt)
    k = draw(rng, shp(layout, B, Hkv, Tkv, D), dt)
    v = draw(rng, shp(layout, B, Hkv, Tkv, D), dt)
    do = draw(rng, shp(layout, B, Hq, Tq, D), dt)
    omask = gmask = mask
    if mask == "additive":
        m = torch.from_numpy(rng.standard_normal((1, Hq, Tq, Tkv), dtype=np.float32)).to(torch.bfloat16)
        omask, gmask = {"kind": "additive", "data": np64(m)}, {"kind": "additive", "data": m.cuda()}
    elif mask == "bool":
        m = torch.from_numpy(rng.random((B, Hq, Tq, Tkv)) < 0.7)
        omask, gmask = {"kind": "bool", "data": m.numpy()}, {"kind": "bool", "data": m.cuda()}
    rate, keep, dro = 0.0, None, None
    if drop:
        rate = 0.15
        keep = st.dropout_keep(21, 2, rate, B, Hq, Tq, Tkv)
        dro = {"keep": keep_words_tensor(keep), "rate": rate}
    scale = 1.0 / np.sqrt(D)
    kw = dict(layout=layout, scale=scale, mask=omask, keep=keep, rate=rate)
    fwd = st.sdpa_train_fwd(np64(q), np64(k), np64(v), **kw)
    o = torch.from_numpy(np.ascontiguousarray(fwd["o"], dtype=np.float32)).to(dt)
    lse = torch.from_numpy(fwd["lse"].astype(np.float32))
    dq, dk, dv = gpu.sdpa_backward(q.cuda(), k.cuda(), v.cuda(), o.cuda(), do.cuda(), lse.cuda(), layout=layout,
                                   scale=scale, mask=gmask, dropout=dro,
                                   grad_dtype=torch.float32 if g32 else None)
    torch.cuda.synchronize()
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), **kw)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        e = norm_err(np64(got), ref[name])
        assert e < GTOL[dt], (name, e)
    if isinstance(mask, dict) and mask.get("offset", 0) < 0:       # rows that see no key: exact zeros
        dead = -mask["offset"]
        assert torch.all(dq[:, :, :dead] == 0) if layout == "bhsd" else torch.all(dq[:, :dead] == 0)


def test_backward_is_deterministic(gpu):
    rng = np.random.default_rng(34)
    B, H, T, D = 1, 4, 300, 64
    t = [draw(rng, (B, H, T, D), torch.bfloat16).cuda() for _ in range(4)]
    o, lse = gpu.sdpa(t[0], t[1], t[2], return_lse=True)
    a = gpu.sdpa_backward(t[0], t[1], t[2], o, t[3], lse)
    b = gpu.sdpa_backward(t[0], t[1], t[2], o, t[3], lse)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


BWD_STREAM_CASES = [
    ("plain", 1, 4, 4, 300, 64, None),
    ("gqa", 2, 8, 2, 257, 128, None),
    ("relpos", 2, 3, 3, 256, 64, (16, 16)),
]


@pytest.mark.parametrize("case", BWD_STREAM_CASES, ids=[c[0] for c in BWD_STREAM_CASES])
def test_backward_concurrent_matches_sequential(gpu, case):
    """dK/dV and dQ side by side on two streams give the same bits as one after
    the other, also when the caller works on a stream of its own and uses the
    gradients there at once (the join must order them before that work)."""
    name, B, Hq, Hkv, T, D, grid = case
    rng = np.random.default_rng(44)
    q, do = (draw(rng, (B, Hq, T, D), torch.bfloat16).cuda() for _ in range(2))
    k, v = (draw(rng, (B, Hkv, T, D), torch.bfloat16).cuda() for _ in range(2))
    if grid:
        rh = (0.3 * draw(rng, (2 * grid[0] - 1, D), torch.float32)).to(torch.bfloat16).cuda()
        rw = (0.3 * draw(rng, (2 * grid[1] - 1, D), torch.float32)).to(torch.bfloat16).cuda()
        o, lse = gpu.sdpa_relpos(q, k, v, rh, rw, grid, return_lse=True)
        call = lambda: gpu.sdpa_relpos_backward(q, k, v, o, do, lse, rh, rw, grid)
    else:
        causal = {"kind": "causal", "offset": 0}
        o, lse = gpu.sdpa(q, k, v, return_lse=True, mask=causal)
        call = lambda: gpu.sdpa_backward(q, k, v, o, do, lse, mask=causal)
    torch.cuda.synchronize()
    outs = {}
    try:
        for conc in (0, 1):
            gpu.set_tuning("bwd_concurrent", conc)
            outs[conc] = call()
            torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            torch.cuda._sleep(2_000_000)              # the backward queues behind work on this stream
            got = call()
            snap = [t.clone() for t in got]          # read on the caller's stream right after the call
        torch.cuda.synchronize()
    finally:
        gpu.set_tuning("bwd_concurrent", 1)
    for x, y, z in zip(outs[0], outs[1], snap):
        assert torch.equal(x, y)
        assert torch.equal(x, z)


@pytest.mark.parametrize("case", [BWD_STREAM_CASES[0], BWD_STREAM_CASES[2]], ids=["plain", "relpos"])
def test_backward_in_graph_matches_eager(gpu, case):
    """A backward call captured into a graph keeps its kernels on the
    capturing stream; every replay, with eager calls (which do use the second
    stream) in between, gives the eager call's bits."""
    name, B, Hq, Hkv, T, D, grid = case
    rng = np.random.default_rng(45)
    q, do = (draw(rng, (B, Hq, T, D), torch.bfloat16).cuda() for _ in range(2))
    k, v = (draw(rng, (B, Hkv, T, D), torch.bfloat16).cuda() for _ in range(2))
    if grid:
        rh = (0.3 * draw(rng, (2 * grid[0] - 1, D), torch.float32)).to(torch.bfloat16).cuda()
        rw = (0.3 * draw(rng, (2 * grid[1] - 1, D), torch.float32)).to(torch.bfloat16).cuda()
        o, lse = gpu.sdpa_relpos(q, k, v, rh, rw, grid, return_lse=True)
        call = lambda: gpu.sdpa_relpos_backward(q, k, v, o, do, lse, rh, rw, grid)
    else:
        o, lse = gpu.sdpa(q, k, v, return_lse=True)
        call = lambda: gpu.sdpa_backward(q, k, v, o, do, lse)
    eager = call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                       # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = call()
    for _ in range(3):
        for t in captured:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(eager, captured):
            assert torch.equal(x, y)
        again = call()                               # eager work between replays
        torch.cuda.synchronize()
        for x, y in zip(eager, again):
            assert torch.equal(x, y)


def test_backward_after_library_forward(gpu):
    """End to end on the GPU: forward with dropout (library keep bits), then the
    backward from the library's own O and lse, against the oracle on the same bits."""
    rng = np.random.default_rng(35)
    B, Hq, Hkv, T, D = 1, 4, 2, 257, 64
    q, k, v, do = (draw(rng, (B, H, T, D), torch.bfloat16) for H in (Hq, Hkv, Hkv, Hq))
    rate = 0.1
    keep_g = gpu.dropout_mask(77, 5, rate, B, Hq, T, T)
    dro = {"keep": keep_g, "rate": rate}
    o, lse = gpu.sdpa(q.cuda(), k.cuda(), v.cuda(), return_lse=True, dropout=dro)
    dq, dk, dv = gpu.sdpa_backward(q.cuda(), k.cuda(), v.cuda(), o, do.cuda(), lse, dropout=dro)
    torch.cuda.synchronize()
    keep = st.dropout_keep(77, 5, rate, B, Hq, T, T)
    assert np.array_equal(keep_g.cpu().numpy().view(np.uint32), st.pack_keep_words(keep))
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), keep=keep, rate=rate)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert norm_err(np64(got), ref[name]) < GTOL[torch.bfloat16], name


def test_backward_rejects_unsupported(gpu):
    x = torch.zeros(1, 1, 8, 16, device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8, device="cuda")
    with pytest.raises(gpu.SdpaError):
        gpu.sdpa_backward(x, x, x, x, x, lse)                       # head_dim 16 is not built
    y = torch.zeros(1, 1, 8, 64, device="cuda", dtype=torch.float32)
    with pytest.raises(gpu.SdpaError):
        gpu.sdpa_backward(y, y, y, y, y, lse)                       # fp32 inputs are not built


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gqa_causal", "sam_global_nobias"])
def test_backward_full_size_sampled_heads(gpu, name):
    """Bench-sized shapes in the launch configuration the benchmark times; the
    oracle checks the full gradients of sampled (batch, KV head) groups."""
    import workloads
    if name == "sam_global_nobias":
        wl = workloads.WORKLOADS["sam_global_relpos"].with_(grid=None)
    else:
        wl = workloads.WORKLOADS[name]
    x = workloads.generate(wl, seed=0)
    rng = np.random.default_rng(36)
    do = draw(rng, tuple(x["q"].shape), torch.bfloat16)
    g = {k: v.cuda() for k, v in x.items()}
    o, lse = gpu.sdpa(g["q"], g["k"], g["v"], layout=wl.layout, scale=wl.scale, mask=wl.mask, return_lse=True)
    dq, dk, dv = gpu.sdpa_backward(g["q"], g["k"], g["v"], o, do.cuda(), lse, layout=wl.layout, scale=wl.scale,
                                   mask=wl.mask)
    torch.cuda.synchronize()
    grp = wl.Hq // wl.Hkv
    to_b = (lambda t: t) if wl.layout == "bhsd" else (lambda t: t.permute(0, 2, 1, 3))
    for (b, hk) in [(0, 0), (wl.B - 1, wl.Hkv - 1)]:
        hs = slice(hk * grp, (hk + 1) * grp)
        qs, dos = np64(to_b(x["q"])[b:b + 1, hs]), np64(to_b(do)[b:b + 1, hs])
        ks, vs = np64(to_b(x["k"])[b:b + 1, hk:hk + 1]), np64(to_b(x["v"])[b:b + 1, hk:hk + 1])
        ref = st.sdpa_bwd(qs, ks, vs, dos, scale=wl.scale, mask=wl.mask)
        assert norm_err(np64(to_b(dq.cpu())[b:b + 1, hs]), ref["dq"]) < GTOL[torch.bfloat16]
        assert norm_err(np64(to_b(dk.cpu())[b:b + 1, hk:hk + 1]), ref["dk"]) < GTOL[torch.bfloat16]
        assert norm_err(np64(to_b(dv.cpu())[b:b + 1, hk:hk + 1]), ref["dv"]) < GTOL[torch.bfloat16]


# ---------------------------------------------------------- rel-pos backward --
RELPOS_BWD_CASES = [
    # dtype, layout, B, H, grid, D, grad fp32
    ("bf16", "bhsd", 1, 2, (16, 64), 64, False),      # SAM global rows (64 wide), 16 of them
    ("bf16", "bshd", 2, 3, (14, 14), 64, False),      # SAM windows
    ("fp16", "bhsd", 1, 2, (14, 14), 64, True),
    ("bf16", "bhsd", 1, 2, (8, 8), 32, True),
    ("bf16", "bhsd", 1, 1, (5, 27), 128, False),      # ragged: T = 135
    ("bf16", "bhsd", 1, 2, (40, 24), 64, False),      # grid rows beyond 32: dS sums through LDS
    ("bf16", "bhsd", 1, 2, (5, 64), 64, False),       # 64 wide, 320 keys: half the last 128-key block past the end
    # more LDS-path grids (a side beyond 32, not 64 wide): head_dim 128 and 32, fp16, bshd, B * H > 2
    ("bf16", "bshd", 2, 3, (40, 24), 128, False),
    ("fp16", "bhsd", 2, 2, (33, 20), 32, True),
    ("fp16", "bshd", 1, 3, (24, 40), 64, False),
    ("bf16", "bhsd", 3, 1, (36, 9), 128, True),
    # grouped table products cut into many query slices (split_h = 24, split_w = 6)
    ("bf16", "bhsd", 2, 12, (16, 64), 64, False),
    # the two shapes on which earlier dQ variants gave wrong gradients
    ("bf16", "bshd", 2, 3, (14, 14), 64, False),
    ("bf16", "bhsd", 1, 1, (5, 27), 128, False),
]


@pytest.mark.parametrize("case", RELPOS_BWD_CASES,
                         ids=[f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}-{c[4][0]}x{c[4][1]}-D{c[5]}{'-g32' if c[6] else ''}"
                              for c in RELPOS_BWD_CASES])
def test_relpos_backward_matches_oracle(gpu, case):
    dts, layout, B, H, grid, D, g32 = case
    dt = DT[dts]
    gh, gw = grid
    T = gh * gw
    rng = np.random.default_rng(37)
    q, k, v, do = (draw(rng, shp(layout, B, H, T, D), dt) for _ in range(4))
    rh = (0.3 * draw(rng, (2 * gh - 1, D), torch.float32)).to(dt)
    rw = (0.3 * draw(rng, (2 * gw - 1, D), torch.float32)).to(dt)
    scale = 1.0 / np.sqrt(D)
    rp = {"rel_pos_h": np64(rh), "rel_pos_w": np64(rw), "grid": grid}
    fwd = st.sdpa_train_fwd(np64(q), np64(k), np64(v), layout=layout, scale=scale, rel_pos=rp)
    o = torch.from_numpy(np.ascontiguousarray(fwd["o"], dtype=np.float32)).to(dt)
    lse = torch.from_numpy(fwd["lse"].astype(np.float32))
    dq, dk, dv, drh, drw = gpu.sdpa_relpos_backward(q.cuda(), k.cuda(), v.cuda(), o.cuda(), do.cuda(), lse.cuda(),
                                                    rh.cuda(), rw.cuda(), grid, layout=layout, scale=scale,
                                                    grad_dtype=torch.float32 if g32 else None)
    torch.cuda.synchronize()
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), layout=layout, scale=scale, rel_pos=rp)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("drel_pos_h", drh), ("drel_pos_w", drw)):
        e = norm_err(np64(got), ref[name])
        assert e < GTOL[dt], (name, e)


RELPOS_DROP_CASES = [
    # dtype, layout, B, H, grid, D: forward route (double-buffered kernel for 16-bit head_dim
    # 64 / 128 with grid_w % 4 == 0, else the generic kernel) and backward mode
    ("bf16", "bhsd", 1, 2, (16, 64), 64),      # 64-wide rows: tiled forward, 64-wide backward mode
    ("bf16", "bshd", 2, 3, (14, 14), 64),      # SAM windows: generic forward, grid <= 32 backward
    ("fp16", "bhsd", 1, 2, (20, 12), 128),     # tiled forward at head_dim 128
    ("bf16", "bhsd", 1, 2, (40, 24), 64),      # a side beyond 32: dS sums through LDS in the backward
    ("bf16", "bhsd", 1, 1, (5, 27), 128),      # grid_w 27: generic forward; ragged T = 135
    ("bf16", "bhsd", 1, 2, (8, 8), 32),        # head_dim 32: generic forward
]


def _relpos_drop_inputs(case, seed):
    dts, layout, B, H, grid, D = case
    dt = DT[dts]
    gh, gw = grid
    T = gh * gw
    rng = np.random.default_rng(seed)
    q, k, v, do = (draw(rng, shp(layout, B, H, T, D), dt) for _ in range(4))
    rh = (0.3 * draw(rng, (2 * gh - 1, D), torch.float32)).to(dt)
    rw = (0.3 * draw(rng, (2 * gw - 1, D), torch.float32)).to(dt)
    rate = 0.15
    keep = st.dropout_keep(23, 5, rate, B, H, T, T)
    rp = {"rel_pos_h": np64(rh), "rel_pos_w": np64(rw), "grid": grid}
    return dt, layout, grid, D, q, k, v, do, rh, rw, rate, keep, rp


@pytest.mark.parametrize("case", RELPOS_DROP_CASES,
                         ids=[f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}-{c[4][0]}x{c[4][1]}-D{c[5]}" for c in RELPOS_DROP_CASES])
def test_relpos_dropout_forward_matches_oracle(gpu, case):
    """Attention dropout with the rel-pos bias ([Axon PR 650], description:
    `:dropout_rate` in :train mode; SAM's bias): O = (W * Z) . V against the
    oracle on the same keep bits; lse is that of the undropped scores."""
    dt, layout, grid, D, q, k, v, do, rh, rw, rate, keep, rp = _relpos_drop_inputs(case, 41)
    scale = 1.0 / np.sqrt(D)
    o, lse = gpu.sdpa_relpos(q.cuda(), k.cuda(), v.cuda(), rh.cuda(), rw.cuda(), grid, layout=layout, scale=scale,
                             out_dtype=torch.float32, return_lse=True,
                             dropout={"keep": keep_words_tensor(keep), "rate": rate})
    torch.cuda.synchronize()
    tiled = case[0] != "fp32" and D in (64, 128) and grid[1] % 4 == 0
    assert gpu.last_kernel() == ("flash_tiled_kernel" if tiled else "generic_fwd_kernel")
    ref = st.sdpa_train_fwd(np64(q), np64(k), np64(v), layout=layout, scale=scale, rel_pos=rp, keep=keep, rate=rate)
    dts = case[0]
    # as for dropout without the bias: the kept weights' factor 65536 / (65536 - thresh) scales the error
    assert max_err(np64(o), ref["o"]) < TOL[dts] * (65536.0 / (65536.0 - round(rate * 65536)))
    assert max_err(np64(lse), ref["lse"]) <= TOL[dts]


@pytest.mark.parametrize("case", RELPOS_DROP_CASES,
                         ids=[f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}-{c[4][0]}x{c[4][1]}-D{c[5]}" for c in RELPOS_DROP_CASES])
def test_relpos_dropout_backward_matches_oracle(gpu, case):
    """Gradients of dropout with the rel-pos bias: dq, dk, dv and both tables'
    gradients against the oracle, the forward pass's O and lse from the oracle."""
    dt, layout, grid, D, q, k, v, do, rh, rw, rate, keep, rp = _relpos_drop_inputs(case, 43)
    scale = 1.0 / np.sqrt(D)
    kw = dict(layout=layout, scale=scale, rel_pos=rp, keep=keep, rate=rate)
    fwd = st.sdpa_train_fwd(np64(q), np64(k), np64(v), **kw)
    o = torch.from_numpy(np.ascontiguousarray(fwd["o"], dtype=np.float32)).to(dt)
    lse = torch.from_numpy(fwd["lse"].astype(np.float32))
    dq, dk, dv, drh, drw = gpu.sdpa_relpos_backward(q.cuda(), k.cuda(), v.cuda(), o.cuda(), do.cuda(), lse.cuda(),
                                                    rh.cuda(), rw.cuda(), grid, layout=layout, scale=scale,
                                                    dropout={"keep": keep_words_tensor(keep), "rate": rate})
    torch.cuda.synchronize()
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), **kw)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("drel_pos_h", drh), ("drel_pos_w", drw)):
        e = norm_err(np64(got), ref[name])
        assert e < GTOL[dt], (name, e)


TABLE_KERNEL_CASES = [
    ("bf16", "bhsd", 1, 2, (16, 64), 64),
    ("fp16", "bshd", 2, 3, (14, 14), 64),
    ("bf16", "bhsd", 1, 2, (40, 24), 128),
    ("bf16", "bhsd", 2, 2, (8, 8), 32),
]


@pytest.mark.parametrize("mfma", [1, 0], ids=["tables-mfma", "tables-valu"])
@pytest.mark.parametrize("case", TABLE_KERNEL_CASES,
                         ids=[f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}-{c[4][0]}x{c[4][1]}-D{c[5]}" for c in TABLE_KERNEL_CASES])
def test_relpos_backward_table_kernels(gpu, case, mfma):
    """The tables' gradients from the matrix-core kernel (lines of the grid,
    fp32 products, partial sums added in a fixed order) and from the
    vector-ALU grouped products ("relpos_bwd_mfma" = 0), against the oracle."""
    dts, layout, B, H, grid, D = case
    dt = DT[dts]
    gh, gw = grid
    T = gh * gw
    rng = np.random.default_rng(47)
    q, k, v, do = (draw(rng, shp(layout, B, H, T, D), dt) for _ in range(4))
    rh = (0.3 * draw(rng, (2 * gh - 1, D), torch.float32)).to(dt)
    rw = (0.3 * draw(rng, (2 * gw - 1, D), torch.float32)).to(dt)
    scale = 1.0 / np.sqrt(D)
    rp = {"rel_pos_h": np64(rh), "rel_pos_w": np64(rw), "grid": grid}
    fwd = st.sdpa_train_fwd(np64(q), np64(k), np64(v), layout=layout, scale=scale, rel_pos=rp)
    o = torch.from_numpy(np.ascontiguousarray(fwd["o"], dtype=np.float32)).to(dt)
    lse = torch.from_numpy(fwd["lse"].astype(np.float32))
    gpu.set_tuning("relpos_bwd_mfma", mfma)
    try:
        dq, dk, dv, drh, drw = gpu.sdpa_relpos_backward(q.cuda(), k.cuda(), v.cuda(), o.cuda(), do.cuda(),
                                                        lse.cuda(), rh.cuda(), rw.cuda(), grid, layout=layout,
                                                        scale=scale)
        torch.cuda.synchronize()
    finally:
        gpu.set_tuning("relpos_bwd_mfma", 1)
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), layout=layout, scale=scale, rel_pos=rp)
    for name, got in (("dq", dq), ("drel_pos_h", drh), ("drel_pos_w", drw)):
        e = norm_err(np64(got), ref[name])
        assert e < GTOL[dt], (name, e)


TERMS_KERNEL_CASES = [
    # dtype, layout, B, H, grid, D
    ("bf16", "bhsd", 1, 2, (16, 64), 64),     # blocks within one 64-wide grid row
    ("bf16", "bshd", 2, 3, (14, 14), 64),     # blocks across rows (windows)
    ("fp16", "bhsd", 1, 2, (5, 27), 128),     # ragged last block
    ("bf16", "bhsd", 2, 2, (40, 24), 32),
    ("fp16", "bshd", 1, 3, (24, 40), 64),
]


@pytest.mark.parametrize("case", TERMS_KERNEL_CASES,
                         ids=[f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}-{c[4][0]}x{c[4][1]}-D{c[5]}" for c in TERMS_KERNEL_CASES])
def test_relpos_backward_with_either_terms_kernel(gpu, case):
    """The rel-pos backward recomputes the terms with relpos_terms: with the
    matrix-core terms kernel and with the vector one, both match the oracle,
    and the fp32 dq of the two agree to u, the 16-bit type's unit roundoff
    (2^-8 bf16, 2^-11 fp16), of its largest value: the two kernels' fp32
    sums differ only in order, which can move a probability across a 16-bit
    rounding boundary before the products."""
    dts, layout, B, H, grid, D = case
    dt = DT[dts]
    gh, gw = grid
    T = gh * gw
    rng = np.random.default_rng(41)
    q, k, v, do = (draw(rng, shp(layout, B, H, T, D), dt) for _ in range(4))
    rh = (0.3 * draw(rng, (2 * gh - 1, D), torch.float32)).to(dt)
    rw = (0.3 * draw(rng, (2 * gw - 1, D), torch.float32)).to(dt)
    scale = 1.0 / np.sqrt(D)
    rp = {"rel_pos_h": np64(rh), "rel_pos_w": np64(rw), "grid": grid}
    fwd = st.sdpa_train_fwd(np64(q), np64(k), np64(v), layout=layout, scale=scale, rel_pos=rp)
    o = torch.from_numpy(np.ascontiguousarray(fwd["o"], dtype=np.float32)).to(dt).cuda()
    lse = torch.from_numpy(fwd["lse"].astype(np.float32)).cuda()
    g = [t.cuda() for t in (q, k, v, do, rh, rw)]
    outs = {}
    try:
        for mf in (1, 0):
            gpu.set_tuning("relpos_mfma", mf)
            outs[mf] = gpu.sdpa_relpos_backward(g[0], g[1], g[2], o, g[3], lse, g[4], g[5], grid, layout=layout,
                                                scale=scale, grad_dtype=torch.float32)
            torch.cuda.synchronize()
    finally:
        gpu.set_tuning("relpos_mfma", 1)
    u = 2.0 ** -8 if dt == torch.bfloat16 else 2.0 ** -11
    assert norm_err(np64(outs[1][0]), np64(outs[0][0])) < u
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), layout=layout, scale=scale, rel_pos=rp)
    for mf in (1, 0):
        for j, name in enumerate(("dq", "dk", "dv", "drel_pos_h", "drel_pos_w")):
            assert norm_err(np64(outs[mf][j]), ref[name]) < GTOL[dt], (mf, name)


def test_relpos_backward_after_library_forward(gpu):
    """The library's own forward (fused terms) feeding its backward, SAM window shape."""
    rng = np.random.default_rng(38)
    B, H, grid, D = 2, 2, (14, 14), 64
    T = grid[0] * grid[1]
    q, k, v, do = (draw(rng, (B, H, T, D), torch.bfloat16) for _ in range(4))
    rh = (0.3 * draw(rng, (27, D), torch.float32)).to(torch.bfloat16)
    rw = (0.3 * draw(rng, (27, D), torch.float32)).to(torch.bfloat16)
    g = [t.cuda() for t in (q, k, v, do, rh, rw)]
    o, lse = gpu.sdpa_relpos(g[0], g[1], g[2], g[4], g[5], grid, return_lse=True)
    out = gpu.sdpa_relpos_backward(g[0], g[1], g[2], o, g[3], lse, g[4], g[5], grid)
    again = gpu.sdpa_relpos_backward(g[0], g[1], g[2], o, g[3], lse, g[4], g[5], grid)
    torch.cuda.synchronize()
    for x, y in zip(out, again):
        assert torch.equal(x, y)                     # deterministic
    rp = {"rel_pos_h": np64(rh), "rel_pos_w": np64(rw), "grid": grid}
    ref = st.sdpa_bwd(np64(q), np64(k), np64(v), np64(do), rel_pos=rp)
    for name, got in zip(("dq", "dk", "dv", "drel_pos_h", "drel_pos_w"), out):
        assert norm_err(np64(got), ref[name]) < GTOL[torch.bfloat16], name


@pytest.mark.slow
def test_relpos_backward_full_size_sampled_heads(gpu):
    """SAM ViT-B global attention at full size in the launch configuration the
    benchmark times: dq, dk, dv of two heads, and both table gradients (which
    sum over every head, so the oracle runs all twelve heads one at a time)
    against the oracle."""
    import workloads
    wl = workloads.WORKLOADS["sam_global_relpos"]
    x = workloads.generate(wl, seed=0)
    rng = np.random.default_rng(39)
    do = draw(rng, tuple(x["q"].shape), torch.bfloat16)
    g = {k: v.cuda() for k, v in x.items()}
    o, lse = gpu.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, scale=wl.scale,
                             return_lse=True)
    dq, dk, dv, drh, drw = gpu.sdpa_relpos_backward(g["q"], g["k"], g["v"], o, do.cuda(), lse, g["rel_pos_h"],
                                                    g["rel_pos_w"], wl.grid, scale=wl.scale)
    torch.cuda.synchronize()
    rp = {"rel_pos_h": np64(x["rel_pos_h"]), "rel_pos_w": np64(x["rel_pos_w"]), "grid": wl.grid}
    drh_ref, drw_ref = 0.0, 0.0
    for h in range(wl.Hq):
        sl = slice(h, h + 1)
        ref = st.sdpa_bwd(np64(x["q"][:, sl]), np64(x["k"][:, sl]), np64(x["v"][:, sl]), np64(do[:, sl]),
                          scale=wl.scale, rel_pos=rp)
        drh_ref = drh_ref + ref["drel_pos_h"]
        drw_ref = drw_ref + ref["drel_pos_w"]
        if h in (0, wl.Hq - 1):
            assert norm_err(np64(dq[:, sl]), ref["dq"]) < GTOL[torch.bfloat16]
            assert norm_err(np64(dk[:, sl]), ref["dk"]) < GTOL[torch.bfloat16]
            assert norm_err(np64(dv[:, sl]), ref["dv"]) < GTOL[torch.bfloat16]
    assert norm_err(np64(drh), drh_ref) < GTOL[torch.bfloat16]
    assert norm_err(np64(drw), drw_ref) < GTOL[torch.bfloat16]
