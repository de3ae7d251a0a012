"""GPU edge cases and invariants: ragged sizes, every mask kind with
broadcast strides and offsets, fully masked rows, GQA ratios, non-default
scale, head_dims, both output dtypes, determinism, and the equivalences the
pages state (rel-pos bias == the same bias passed as an additive mask)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL, max_err, np64

pytestmark = pytest.mark.gpu


def rnd(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def layout_shape(B, H, T, D, layout):
    return (B, H, T, D) if layout == "bhsd" else (B, T, H, D)


def check(fa, B, Hq, Hkv, Tq, Tkv, D, *, dtype=torch.bfloat16, layout="bhsd", mask=None, scale=None, seed=0,
          omask=None):
    q = rnd(layout_shape(B, Hq, Tq, D, layout), dtype, seed)
    k = rnd(layout_shape(B, Hkv, Tkv, D, layout), dtype, seed + 1)
    v = rnd(layout_shape(B, Hkv, Tkv, D, layout), dtype, seed + 2)
    gm = None
    if mask is not None and "data" in mask:
        gm = dict(mask, data=mask["data"].cuda())
    elif mask is not None:
        gm = mask
    o, lse = fa.sdpa(q.cuda(), k.cuda(), v.cuda(), layout=layout, scale=scale, mask=gm, out_dtype=torch.float32,
                     return_lse=True)
    torch.cuda.synchronize()
    om = omask if omask is not None else mask
    if om is not None and "data" in om:
        om = dict(om, data=np64(om["data"]) if om["data"].dtype != torch.bool else om["data"].numpy())
    ref = oracle.sdpa(np64(q), np64(k), np64(v), layout=layout, scale=scale, mask=om)
    tol = TOL["fp32" if dtype == torch.float32 else "bf16"]
    err = max_err(np64(o), ref["o"])
    assert err <= tol, f"max-abs {err:.3e}"
    rl, gl = ref["lse"], np64(lse)
    assert np.array_equal(np.isneginf(rl), np.isneginf(gl))
    fin = np.isfinite(rl)
    assert max_err(gl[fin], rl[fin]) <= tol
    return o


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Tq,Tkv", [(1, 1), (1, 200), (77, 1), (33, 65), (130, 257), (256, 64)])
def test_ragged_sizes(gpu, D, Tq, Tkv):
    check(gpu, 2, 2, 2, Tq, Tkv, D, seed=Tq * 7 + Tkv)


@pytest.mark.parametrize("ratio", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_gqa_ratios(gpu, ratio, layout):
    check(gpu, 2, 8, 8 // ratio, 97, 150, 64, layout=layout, seed=ratio)


@pytest.mark.parametrize("offset", [0, 5, -7, -200])
@pytest.mark.parametrize("D", [64, 128])
def test_causal_offsets(gpu, offset, D):
    check(gpu, 1, 4, 1, 150, 190, D, mask={"kind": "causal", "offset": offset}, seed=3)


@pytest.mark.parametrize("w,offset", [(1, 0), (7, 0), (64, 3), (100, -5), (1000, 0)])
def test_sliding(gpu, w, offset):
    check(gpu, 1, 4, 2, 260, 260, 128, layout="bshd", mask={"kind": "sliding", "window": w, "offset": offset}, seed=4)


@pytest.mark.parametrize("mshape", [(2, 4, 70, 130), (1, 1, 70, 130), (2, 1, 1, 130), (1, 4, 70, 1)])
@pytest.mark.parametrize("mdt", [torch.float32, torch.bfloat16])
def test_additive_mask_broadcast(gpu, mshape, mdt):
    m = rnd(mshape, mdt, 9)
    check(gpu, 2, 4, 2, 70, 130, 64, mask={"kind": "additive", "data": m}, seed=5)


def test_bool_mask_with_dead_rows(gpu):
    g = torch.Generator().manual_seed(11)
    m = torch.rand((2, 4, 70, 130), generator=g) < 0.3
    m[0, 1, 5] = False          # a fully masked row: output 0, lse -inf
    check(gpu, 2, 4, 4, 70, 130, 128, mask={"kind": "bool", "data": m}, seed=6)


def test_non_default_scale_and_fp32(gpu):
    check(gpu, 1, 2, 2, 100, 90, 64, scale=0.37, seed=7)
    check(gpu, 1, 2, 1, 100, 90, 40, dtype=torch.float32, scale=0.2, seed=8)
    check(gpu, 1, 2, 2, 50, 90, 16, scale=0.9, seed=9)
    check(gpu, 1, 2, 2, 50, 90, 32, seed=10, mask={"kind": "causal", "offset": 40})


def test_bf16_output_rounding(gpu):
    q, k, v = (rnd((1, 2, 96, 64), torch.bfloat16, s).cuda() for s in (1, 2, 3))
    o32 = gpu.sdpa(q, k, v, out_dtype=torch.float32)
    o16 = gpu.sdpa(q, k, v)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_deterministic(gpu):
    wl = workloads.replica("gqa_causal")
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=1).items()}
    a = gpu.sdpa(x["q"], x["k"], x["v"], layout=wl.layout, mask=wl.mask)
    b = gpu.sdpa(x["q"], x["k"], x["v"], layout=wl.layout, mask=wl.mask)
    assert torch.equal(a, b)


def test_gqa_equals_repeated_kv(gpu):
    q, k, v = (rnd(s, torch.bfloat16, i).cuda() for i, s in enumerate([(1, 8, 70, 64), (1, 2, 90, 64), (1, 2, 90, 64)]))
    a = gpu.sdpa(q, k, v, out_dtype=torch.float32)
    b = gpu.sdpa(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(),
                 out_dtype=torch.float32)
    assert max_err(np64(a), np64(b)) <= 1e-6


def test_relpos_equals_additive_route(gpu):
    """The rel-pos bias injected from term rows matches the same bias passed as
    an additive [B, H, T, T] mask (mlx-examples issue 1451, body)."""
    wl = workloads.replica("sam_global_relpos")
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=2).items()}
    o1 = gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid, scale=wl.scale,
                         out_dtype=torch.float32)
    th, tw = gpu.relpos_terms(x["q"], x["rel_pos_h"], x["rel_pos_w"], wl.grid)
    gh, gw = wl.grid
    j = torch.arange(gh * gw, device="cuda")
    bias = (th[..., j // gw] + tw[..., j % gw]).contiguous()
    o2 = gpu.sdpa(x["q"], x["k"], x["v"], scale=wl.scale, mask={"kind": "additive", "data": bias},
                  out_dtype=torch.float32)
    # Both routes round P to bf16; the bias enters the fp32 scores at different
    # points (accumulator initialisation vs an added mask), which can flip the
    # rounding of single P entries (2^-9 relative), so agreement is ~1e-4.
    assert max_err(np64(o1), np64(o2)) <= 1e-3


def test_windowed_equals_independent_windows(gpu):
    wl = workloads.WORKLOADS["sam_window_relpos"]
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=0).items()}
    o = gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid, scale=wl.scale,
                        out_dtype=torch.float32)
    for wdx in (0, 7, 24):
        s = slice(wdx, wdx + 1)
        o1 = gpu.sdpa_relpos(x["q"][s].contiguous(), x["k"][s].contiguous(), x["v"][s].contiguous(),
                             x["rel_pos_h"], x["rel_pos_w"], wl.grid, scale=wl.scale, out_dtype=torch.float32)
        assert torch.equal(o1, o[s])
    # the last window is mostly zero padding: a padded query (q = 0) has zero
    # scores and zero rel-pos terms, so its output is the mean of the window's V
    last = x["v"][24].float().mean(dim=1)      # [H, D]
    assert max_err(np64(o[24, :, 195]), np64(last)) <= 1e-3


@pytest.mark.parametrize("B,dtype,layout", [(22, "bf16", "bhsd"), (26, "bf16", "bhsd"), (27, "bf16", "bhsd"),
                                            (26, "fp16", "bshd")])
def test_window_balanced_launch(gpu, B, dtype, layout):
    """More (window, head) items than CUs: 264 and 312 items take the balanced
    launch (one workgroup per CU, the items past the first 256 spread over the
    workgroups two query blocks at a time), 324 the one-workgroup-per-item
    launch.  Every window's output equals that window computed alone (one
    workgroup per item, the same per-wave arithmetic), and sampled rows match
    the oracle; also in fp16 and the bshd layout."""
    from parity_util import rows_of, sample_picks
    wl = workloads.WORKLOADS["sam_window_relpos"].with_(B=B, window_image=None, dtype=dtype, layout=layout)
    x = workloads.generate(wl, seed=B)
    g = {k_: t.cuda() for k_, t in x.items()}
    o, lse = gpu.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=layout,
                             scale=wl.scale, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_window_kernel"
    for wdx in sorted({0, 1, B // 2, B - 2, B - 1}):
        s = slice(wdx, wdx + 1)
        o1 = gpu.sdpa_relpos(g["q"][s].contiguous(), g["k"][s].contiguous(), g["v"][s].contiguous(),
                             g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=layout, scale=wl.scale,
                             out_dtype=torch.float32)
        assert torch.equal(o1, o[s]), wdx
    picks = sample_picks(wl, n_random=24, seed=B)
    picks += [(b, h, i) for b in (B - 1, B - 2) for h in (0, 11) for i in (0, 100, 191, 192, 195)]
    rp = {"rel_pos_h": np64(x["rel_pos_h"]), "rel_pos_w": np64(x["rel_pos_w"]), "grid": wl.grid}
    ro, rl = oracle.sdpa_rows(np64(x["q"]), np64(x["k"]), np64(x["v"]), picks, layout=layout, scale=wl.scale,
                              rel_pos=rp)
    assert max_err(np64(rows_of(o, picks, layout)), ro) <= TOL[dtype]
    assert max_err(np64(torch.stack([lse[b, h, i] for b, h, i in picks])), rl) <= TOL[dtype]


def test_first_causal_row_is_v0(gpu):
    wl = workloads.WORKLOADS["gqa_causal"]
    x = {k_: t.cuda() for k_, t in workloads.generate(wl.with_(B=1), seed=0).items()}
    o = gpu.sdpa(x["q"], x["k"], x["v"], layout="bshd", mask=wl.mask, out_dtype=torch.float32)
    v0 = x["v"][:, 0].float().repeat_interleave(4, dim=1)   # [B, Hq, D]
    assert max_err(np64(o[:, 0]), np64(v0)) <= 1e-6


@pytest.mark.parametrize("name", ["sam_global_relpos", "sam_window_relpos"])
def test_relpos_fused_equals_unfused(gpu, name):
    """The single-kernel rel-pos path (terms formed in the attention kernel) and
    the two-kernel path (relpos_terms into the workspace) agree.  For the global
    grid both routes run the same matrix-core kernel (bf16 probabilities), so
    only the order of term arithmetic differs (1e-3).  For windows the unfused
    route runs the fp32 vector kernel: the fused kernel's bf16 rounding of each
    probability (relative 2^-9) moves an output by at most 2^-9 * max|v|."""
    wl = workloads.replica(name)
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=4).items()}
    args = (x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid)
    a = gpu.sdpa_relpos(*args, scale=wl.scale, out_dtype=torch.float32)
    gpu.set_tuning("relpos_fused", 0)
    try:
        b = gpu.sdpa_relpos(*args, scale=wl.scale, out_dtype=torch.float32)
    finally:
        gpu.set_tuning("relpos_fused", 1)
    tol = 1e-3 if name == "sam_global_relpos" else 2.0 ** -9 * float(x["v"].float().abs().max()) + 1e-4
    assert max_err(np64(a), np64(b)) <= tol
    ref = oracle.sdpa(np64(x["q"].cpu()), np64(x["k"].cpu()), np64(x["v"].cpu()), scale=wl.scale,
                      rel_pos={"rel_pos_h": np64(x["rel_pos_h"].cpu()), "rel_pos_w": np64(x["rel_pos_w"].cpu()),
                               "grid": wl.grid})
    assert max_err(np64(a), ref["o"]) <= TOL["bf16"]
    assert max_err(np64(b), ref["o"]) <= TOL["bf16"]


@pytest.mark.parametrize("splits", [1, 2, 5, 32, 0])
def test_d16_split_kv_invariance(gpu, splits):
    """Few queries against a long key range: any split-KV chunk count merges
    (by log-sum-exp) to the same attention."""
    gpu.set_tuning("num_splits", splits)
    try:
        check(gpu, 1, 8, 8, 7, 4096, 16, scale=0.25, seed=12)
        check(gpu, 2, 6, 3, 5, 1000, 16, layout="bshd", seed=13, mask={"kind": "causal", "offset": 600})
    finally:
        gpu.set_tuning("num_splits", 0)


TILED_SPLIT_CASES = [
    # (B, Hq, Hkv, Tq, Tkv, layout, mask): decode-like shapes on the double-buffered kernel
    (1, 8, 2, 1, 4096, "bhsd", None),                                            # 4 heads per workgroup
    (2, 4, 4, 5, 1000, "bshd", {"kind": "causal", "offset": 995}),               # one head per workgroup
    (1, 6, 3, 33, 3001, "bhsd", {"kind": "sliding", "window": 700, "offset": 2968}),   # chunks outside the window
    (1, 4, 2, 3, 700, "bhsd", {"kind": "causal", "offset": -1}),                 # row 0 has no allowed key
]


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 0])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_tiled_split_kv_invariance(gpu, splits, D, dtype):
    """Head_dim 64 / 128 split-KV: the key range cut into 1 .. 64 chunks (0 =
    the automatic count), each chunk's (max, sum, unnormalised O) merged by
    log-sum-exp, gives the attention and the log-sum-exp of the oracle; rows
    with no allowed key stay O = 0, lse = -inf."""
    gpu.set_tuning("num_splits", splits)
    try:
        for i, (B, Hq, Hkv, Tq, Tkv, layout, mask) in enumerate(TILED_SPLIT_CASES):
            check(gpu, B, Hq, Hkv, Tq, Tkv, D, dtype=dtype, layout=layout, mask=mask, seed=40 + i)
            if splits != 1:
                assert gpu.last_kernel() == "flash_tiled_kernel"
    finally:
        gpu.set_tuning("num_splits", 0)


def test_tiled_split_kv_automatic_and_deterministic(gpu):
    """A decode shape takes the split route by itself (the workspace query
    says so), and two calls give bit-identical output and log-sum-exp (the
    chunks merge in a fixed order)."""
    lib = gpu.load()
    B, Hq, Hkv, Tq, Tkv, D = 1, 32, 8, 1, 8192, 128
    assert lib.sdpa_workspace_size(1, B, Hq, Hkv, Tq, Tkv, D, float("nan"), 0, 0, 0) > 0
    q, k, v = (rnd(s, torch.bfloat16, 50 + j).cuda()
               for j, s in enumerate([(B, Hq, Tq, D), (B, Hkv, Tkv, D), (B, Hkv, Tkv, D)]))
    o1, l1 = gpu.sdpa(q, k, v, out_dtype=torch.float32, return_lse=True)
    assert gpu.last_kernel() == "flash_tiled_kernel"
    o2, l2 = gpu.sdpa(q, k, v, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref = oracle.sdpa(np64(q), np64(k), np64(v))
    assert max_err(np64(o1), ref["o"]) <= TOL["bf16"]
    assert max_err(np64(l1), ref["lse"]) <= TOL["bf16"]


def test_tiled_split_kv_tensor_mask_runs_unsplit(gpu):
    """A forced chunk count with a tensor mask at head_dim 64: the split route
    does not take tensor masks, so the call runs unsplit and stays exact."""
    g = torch.Generator().manual_seed(51)
    m = torch.rand((1, 4, 3, 2000), generator=g) < 0.7
    gpu.set_tuning("num_splits", 8)
    try:
        check(gpu, 1, 4, 4, 3, 2000, 64, mask={"kind": "bool", "data": m}, seed=52)
    finally:
        gpu.set_tuning("num_splits", 0)


@pytest.mark.parametrize("Tkv", [1, 7, 8, 9, 33, 64])
def test_d16_key_packing(gpu, Tkv):
    check(gpu, 1, 8, 8, 300, Tkv, 16, scale=0.25, seed=14)
    check(gpu, 2, 6, 2, 70, Tkv, 16, layout="bshd", seed=15)


def test_d16_masks(gpu):
    g = torch.Generator().manual_seed(16)
    m = torch.rand((1, 8, 7, 500), generator=g) < 0.5
    check(gpu, 1, 8, 8, 7, 500, 16, mask={"kind": "bool", "data": m}, seed=17)
    a = rnd((1, 1, 100, 9), torch.float32, 18)
    check(gpu, 1, 8, 4, 100, 9, 16, mask={"kind": "additive", "data": a}, seed=19)
    check(gpu, 1, 4, 4, 100, 50, 16, mask={"kind": "sliding", "window": 5, "offset": -40}, seed=20)


def _split_mode(gpu, mode):
    """0: one key range per wave; 1: key halves in 4-wave workgroups; 2: key
    halves in 12-wave workgroups (forced for any size)."""
    gpu.set_tuning("split_halves", 1 if mode else 0)
    gpu.set_tuning("split_wide", 2 if mode == 2 else 0)


def _split_default(gpu):
    gpu.set_tuning("split_halves", 1)
    gpu.set_tuning("split_wide", 1)


@pytest.mark.parametrize("name", ["sam_global_relpos"])
@pytest.mark.parametrize("halves", [0, 1, 2])
@pytest.mark.parametrize("fused", [0, 1])
@pytest.mark.parametrize("gh", [5, 7])
def test_relpos_kernel_variants(gpu, name, halves, fused, gh):
    """Every kernel route for the SAM global rel-pos shape agrees with the oracle:
    key range split in-workgroup or not (4- or 12-wave workgroups; 5 and 7
    grid rows leave the last 192-row workgroup partly empty), terms formed
    in-kernel or precomputed."""
    wl = workloads.replica(name, grid=(gh, 64), Tq=gh * 64, Tkv=gh * 64)
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=5).items()}
    _split_mode(gpu, halves)
    gpu.set_tuning("relpos_fused", fused)
    try:
        o, lse = gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid, scale=wl.scale,
                                 out_dtype=torch.float32, return_lse=True)
        # with the in-workgroup split off, precomputed terms go to the double-buffered
        # kernel, terms formed in the kernel to the general MFMA kernel
        want = ["flash_mfma_kernel" if fused else "flash_tiled_kernel", "flash_split64_kernel",
                "flash_split64w_kernel"][halves]
        assert gpu.last_kernel() == want
    finally:
        _split_default(gpu)
        gpu.set_tuning("relpos_fused", 1)
    ref = oracle.sdpa(np64(x["q"].cpu()), np64(x["k"].cpu()), np64(x["v"].cpu()), scale=wl.scale,
                      rel_pos={"rel_pos_h": np64(x["rel_pos_h"].cpu()), "rel_pos_w": np64(x["rel_pos_w"].cpu()),
                               "grid": wl.grid})
    assert max_err(np64(o), ref["o"]) <= TOL["bf16"]
    assert max_err(np64(lse), ref["lse"]) <= TOL["bf16"]


@pytest.mark.parametrize("fused", [0, 1])
def test_wide_split_fp16(gpu, fused):
    """The 12-wave workgroups on fp16 inputs with fp16 output."""
    wl = workloads.replica("sam_global_relpos", grid=(7, 64), Tq=7 * 64, Tkv=7 * 64, dtype="fp16")
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=6).items()}
    _split_mode(gpu, 2)
    gpu.set_tuning("relpos_fused", fused)
    try:
        o = gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid, scale=wl.scale)
        assert gpu.last_kernel() == "flash_split64w_kernel"
    finally:
        _split_default(gpu)
        gpu.set_tuning("relpos_fused", 1)
    assert o.dtype == torch.float16
    ref = oracle.sdpa(np64(x["q"].cpu()), np64(x["k"].cpu()), np64(x["v"].cpu()), scale=wl.scale,
                      rel_pos={"rel_pos_h": np64(x["rel_pos_h"].cpu()), "rel_pos_w": np64(x["rel_pos_w"].cpu()),
                               "grid": wl.grid})
    assert max_err(np64(o), ref["o"]) <= TOL["fp16"]


@pytest.mark.parametrize("halves", [0, 1, 2])
@pytest.mark.parametrize("Tkv", [32, 33, 95, 200, 4096])
def test_d64_no_mask_key_splits(gpu, halves, Tkv):
    _split_mode(gpu, halves)
    try:
        check(gpu, 1, 3, 3, 130, Tkv, 64, seed=21)
        check(gpu, 1, 4, 2, 64, Tkv, 64, layout="bshd", seed=22)
        check(gpu, 2, 2, 1, 400, Tkv, 64, seed=23)
    finally:
        _split_default(gpu)


@pytest.mark.parametrize("pattern", ["rising", "falling", "spike", "huge"])
@pytest.mark.parametrize("D", [64, 128])
def test_running_max_paths(gpu, pattern, D):
    """Score patterns that move the running max: scores rising across key tiles
    (rescale on almost every tile), falling (probabilities far below the
    reference), one dominant late key, and logits of +-200 that would overflow
    exp2 against a stale reference."""
    T = 700
    g = torch.Generator().manual_seed(31)
    q = torch.randn((1, 2, 65, D), generator=g)
    k = torch.randn((1, 2, T, D), generator=g) * 0.1
    v = torch.randn((1, 2, T, D), generator=g)
    ramp = torch.linspace(0, 1, T).view(1, 1, T, 1)
    if pattern == "rising":
        k = k + ramp * q.mean(dim=2, keepdim=True) * 3
    elif pattern == "falling":
        k = k + (1 - ramp) * q.mean(dim=2, keepdim=True) * 3
    elif pattern == "spike":
        k[:, :, 650] = q.mean(dim=2) * 2
    else:
        k = k * 40.0
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    ref = oracle.sdpa(np64(q), np64(k), np64(v), scale=1.0 / D ** 0.5)
    for halves, tiled in ((0, 0), (0, 1), (1, 1), (2, 1)):
        _split_mode(gpu, halves)
        gpu.set_tuning("tiled", tiled)
        try:
            o = gpu.sdpa(q.cuda(), k.cuda(), v.cuda(), scale=1.0 / D ** 0.5, out_dtype=torch.float32)
        finally:
            _split_default(gpu)
            gpu.set_tuning("tiled", 1)
        assert max_err(np64(o), ref["o"]) <= TOL["bf16"], (pattern, halves, tiled)


@pytest.mark.parametrize("tiled", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", [None, {"kind": "causal", "offset": 0}, {"kind": "causal", "offset": 37},
                                  {"kind": "sliding", "window": 45, "offset": -3}])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (6, 3), (3, 3)])
def test_long_range_kernels(gpu, tiled, D, mask, Hq, Hkv):
    """The double-buffered kernel (4, 2 or 1 query heads per workgroup sharing
    a KV head) and the general MFMA kernel on the same masked, ragged inputs:
    several query blocks, key tiles skipped outside the band, partial tiles on
    both band edges and at the end of the key range."""
    gpu.set_tuning("split_halves", 0)
    gpu.set_tuning("tiled", tiled)
    try:
        for layout in ("bhsd", "bshd"):
            check(gpu, 2, Hq, Hkv, 261, 299, D, layout=layout, mask=mask, seed=D + Hq)
    finally:
        gpu.set_tuning("split_halves", 1)
        gpu.set_tuning("tiled", 1)


@pytest.mark.parametrize("scale", [-0.125, 0.0])
@pytest.mark.parametrize("mask", [None, {"kind": "causal", "offset": 0}])
def test_non_positive_scale(gpu, scale, mask):
    """A negative scale flips which key scores highest; a zero scale averages
    the allowed values.  Both follow the plain definition."""
    check(gpu, 1, 4, 2, 70, 90, 64, mask=mask, scale=scale, seed=11)
    check(gpu, 1, 4, 2, 70, 90, 128, mask=mask, scale=scale, seed=12)


def test_relpos_non_positive_scale(gpu):
    """Rel-pos attention with a negative scale runs the two-launch route and
    still matches the definition (the bias itself is never scaled)."""
    wl = workloads.replica("sam_global_relpos", B=1, Hq=2, Hkv=2, Tq=192, Tkv=192, grid=(3, 64), scale=-0.2)
    x = workloads.generate(wl, seed=5, layout="bhsd")
    g = {k: v.cuda() for k, v in x.items()}
    o = gpu.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, scale=wl.scale,
                        out_dtype=torch.float32)
    ref = oracle.sdpa(np64(x["q"]), np64(x["k"]), np64(x["v"]), scale=wl.scale,
                      rel_pos={"rel_pos_h": np64(x["rel_pos_h"]), "rel_pos_w": np64(x["rel_pos_w"]), "grid": wl.grid})
    assert max_err(np64(o), ref["o"]) <= TOL["bf16"]



TILED_RELPOS_CASES = [
    # (B, H, grid, D, layout): rel-pos with precomputed terms on the double-buffered kernel
    (1, 2, (64, 64), 128, "bhsd"),      # SAM's global grid at head_dim 128
    (2, 3, (32, 32), 64, "bshd"),       # the grid of a 512-pixel image
    (1, 2, (20, 12), 128, "bhsd"),      # grid_w not dividing the 32-key tile: tiles span grid rows
    (2, 2, (7, 4), 64, "bhsd"),         # grid_w 4: eight grid rows per key tile, T = 28 (one partial tile)
    (1, 3, (9, 36), 128, "bshd"),       # T = 324: ragged last tile
]


@pytest.mark.parametrize("case", TILED_RELPOS_CASES, ids=lambda c: f"B{c[0]}H{c[1]}g{c[2][0]}x{c[2][1]}D{c[3]}{c[4]}")
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_tiled_relpos_grids(gpu, case, dtype):
    """Rel-pos at head_dim 128 and on grids other than the fused kernels' (any
    grid_w that is a multiple of 4): relpos_terms into the workspace, then the
    double-buffered matrix-core kernel reads each key tile's terms.  Tables of
    standard deviation 0.1 make the bias move the softmax (|bias| ~ 1)."""
    B, H, (gh, gw), D, layout = case
    T = gh * gw
    assert not gpu.relpos_fused(dtype, D, (gh, gw))
    q = rnd(layout_shape(B, H, T, D, layout), dtype, 60)
    k = rnd(layout_shape(B, H, T, D, layout), dtype, 61)
    v = rnd(layout_shape(B, H, T, D, layout), dtype, 62)
    rh = (rnd((2 * gh - 1, D), torch.float32, 63) * 0.1).to(dtype)
    rw = (rnd((2 * gw - 1, D), torch.float32, 64) * 0.1).to(dtype)
    o, lse = gpu.sdpa_relpos(q.cuda(), k.cuda(), v.cuda(), rh.cuda(), rw.cuda(), (gh, gw), layout=layout,
                             out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_tiled_kernel"
    ref = oracle.sdpa(np64(q), np64(k), np64(v), layout=layout,
                      rel_pos={"rel_pos_h": np64(rh), "rel_pos_w": np64(rw), "grid": (gh, gw)})
    tol = TOL["bf16" if dtype == torch.bfloat16 else "fp16"]
    assert max_err(np64(o), ref["o"]) <= tol
    assert max_err(np64(lse), ref["lse"]) <= tol


def test_relpos_precomputed_terms_on_general_mfma_kernel(gpu):
    """With the double-buffered kernel and the in-workgroup split switched off,
    precomputed terms on a 64-wide grid run on the general MFMA kernel."""
    wl = workloads.replica("sam_global_relpos", grid=(5, 64), Tq=320, Tkv=320)
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=6).items()}
    _split_mode(gpu, 0)
    gpu.set_tuning("relpos_fused", 0)
    gpu.set_tuning("tiled", 0)
    try:
        o = gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid, scale=wl.scale,
                            out_dtype=torch.float32)
        assert gpu.last_kernel() == "flash_mfma_kernel"
    finally:
        _split_default(gpu)
        gpu.set_tuning("relpos_fused", 1)
        gpu.set_tuning("tiled", 1)
    ref = oracle.sdpa(np64(x["q"].cpu()), np64(x["k"].cpu()), np64(x["v"].cpu()), scale=wl.scale,
                      rel_pos={"rel_pos_h": np64(x["rel_pos_h"].cpu()), "rel_pos_w": np64(x["rel_pos_w"].cpu()),
                               "grid": wl.grid})
    assert max_err(np64(o), ref["o"]) <= TOL["bf16"]

def test_dispatch_names_the_kernel(gpu):
    """Which kernel each workload family reaches (the benchmark and profiles
    name the dominant kernel from this)."""
    def run(Hq, Hkv, Tq, Tkv, D, dtype=torch.bfloat16, mask=None, scale=None):
        q = rnd((1, Hq, Tq, D), dtype, 1).cuda()
        k = rnd((1, Hkv, Tkv, D), dtype, 2).cuda()
        v = rnd((1, Hkv, Tkv, D), dtype, 3).cuda()
        gm = dict(mask, data=mask["data"].cuda()) if mask and "data" in mask else mask
        gpu.sdpa(q, k, v, mask=gm, scale=scale)
        torch.cuda.synchronize()
        return gpu.last_kernel()
    assert run(4, 1, 300, 300, 128, mask={"kind": "causal", "offset": 0}) == "flash_tiled_kernel"
    assert run(2, 2, 300, 300, 64) == "flash_split64_kernel"
    add = {"kind": "additive", "data": rnd((1, 1, 300, 300), torch.float32, 4)}
    assert run(2, 2, 300, 300, 64, mask=add) == "flash_tiled_kernel"
    keyb = {"kind": "additive", "data": rnd((1, 1, 300, 1), torch.float32, 4)}     # broadcast along keys
    assert run(2, 2, 300, 300, 64, mask=keyb) == "flash_mfma_kernel"
    assert run(2, 2, 100, 100, 64, dtype=torch.float32) == "generic_fwd_kernel"
    assert run(8, 8, 7, 500, 16) == "d16_qpack_kernel"
    assert run(8, 8, 500, 7, 16) == "d16_kpack_kernel"
    assert run(2, 2, 100, 100, 64, scale=-1.0) == "generic_fwd_kernel"
    wl = workloads.replica("sam_global_relpos")
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=0, layout="bhsd").items()}
    gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_split64_kernel"
    wl = workloads.WORKLOADS["sam_global_relpos"]              # 256 workgroups of 192 rows: one per CU
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=0, layout="bhsd").items()}
    gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_split64w_kernel"
    wl = workloads.replica("sam_window_relpos")
    x = {k_: t.cuda() for k_, t in workloads.generate(wl, seed=0, layout="bhsd").items()}
    gpu.sdpa_relpos(x["q"], x["k"], x["v"], x["rel_pos_h"], x["rel_pos_w"], wl.grid)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_window_kernel"


def _mask_store(shape, Tkv_store, kind, mdt, seed):
    """Storage for a mask of `shape` (last axis Tkv) with rows Tkv_store wide."""
    full = rnd(shape[:-1] + (Tkv_store,), torch.float32, seed)
    if kind == "bool":
        full = full > -0.5
        full[..., :3] = True
        return full
    return full.to(mdt)


@pytest.mark.parametrize("tiled", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind,mdt", [("additive", torch.float32), ("additive", torch.bfloat16), ("bool", torch.bool)])
@pytest.mark.parametrize("mshape,Tkv_store", [((2, 4, 100, 224), 224), ((1, 1, 100, 201), 208), ((2, 1, 1, 201), 208),
                                              ((1, 4, 100, 201), 208)])
def test_tensor_mask_kernels(gpu, tiled, D, kind, mdt, mshape, Tkv_store):
    """Additive (fp32, bf16) and boolean masks with broadcast strides and rows
    wider than the key range, through the double-buffered kernel (mask blocks
    copied to LDS) and through the general MFMA kernel: both against the oracle."""
    full = _mask_store(mshape, Tkv_store, kind, mdt, seed=D + len(kind))
    Tkv = mshape[-1]
    m, mg = full[..., :Tkv], full.cuda()[..., :Tkv]       # the same strided view on both sides
    assert mg.stride() == m.stride()
    gpu.set_tuning("tiled", tiled)
    try:
        check(gpu, 2, 4, 2, 100, Tkv, D, mask={"kind": kind, "data": mg}, seed=D,
              omask={"kind": kind, "data": m.contiguous()})
    finally:
        gpu.set_tuning("tiled", 1)


@pytest.mark.parametrize("qmul", [1.0, 12.0, 60.0])
def test_window_running_max(gpu, qmul):
    """The 14x14 window kernel's optimistic running max: scaled-up queries give
    logits of tens to hundreds, so tiles past the first must move the reference
    (exact path) or overflow; every case matches the definition."""
    wl = workloads.replica("sam_window_relpos", B=1, Hq=2, Hkv=2)
    x = workloads.generate(wl, seed=9, layout="bhsd")
    x["q"] = (x["q"].float() * qmul).to(torch.bfloat16)
    g = {k_: t.cuda() for k_, t in x.items()}
    o = gpu.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, scale=wl.scale,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_window_kernel"
    ref = oracle.sdpa(np64(x["q"]), np64(x["k"]), np64(x["v"]), scale=wl.scale,
                      rel_pos={"rel_pos_h": np64(x["rel_pos_h"]), "rel_pos_w": np64(x["rel_pos_w"]), "grid": wl.grid})
    assert max_err(np64(o), ref["o"]) <= TOL["bf16"]


GENERIC_CASES = [
    # B, Hq, Hkv, Tq, Tkv, D, dtype, mask
    (1, 2, 2, 64, 64, 16, torch.float32, None),
    (1, 2, 1, 50, 77, 16, torch.float32, None),                     # ragged, GQA
    (2, 3, 3, 130, 17, 8, torch.float32, None),                     # D < 16: element-wise copies; 2 key tiles
    (1, 2, 2, 70, 200, 32, torch.float32, {"kind": "causal", "offset": 5}),
    (1, 2, 2, 70, 200, 24, torch.float32, {"kind": "sliding", "window": 19, "offset": 3}),
    (1, 2, 2, 33, 1, 16, torch.float32, None),                       # one key (one wave)
    (1, 4, 2, 70, 130, 32, torch.float32, "additive"),
    (1, 2, 2, 70, 45, 16, torch.float32, "bool"),
    (1, 2, 2, 70, 150, 40, torch.float32, None),                     # head_dim 40 stays on one wave
]


@pytest.mark.parametrize("waves", [0, 1])
@pytest.mark.parametrize("case", range(len(GENERIC_CASES)))
def test_generic_kernel_wave_split(gpu, waves, case):
    """The vector-ALU kernel with its key range split over four waves (small
    launches, head_dim <= 32) and with one wave: both against the oracle, on
    ragged sizes, every mask family, a single key and head_dim below 16."""
    B, Hq, Hkv, Tq, Tkv, D, dt, mask = GENERIC_CASES[case]
    if mask in ("additive", "bool"):
        g = torch.Generator().manual_seed(40 + case)
        if mask == "additive":
            data = torch.randn((B, 1, Tq, Tkv), generator=g)
        else:
            data = torch.rand((1, Hq, Tq, Tkv), generator=g) > 0.3
            data[..., 0] = True
        mask = {"kind": mask, "data": data}
    gpu.set_tuning("generic_waves", waves)
    try:
        check(gpu, B, Hq, Hkv, Tq, Tkv, D, dtype=dt, mask=mask, seed=30 + case)
        assert gpu.last_kernel() == "generic_fwd_kernel"
    finally:
        gpu.set_tuning("generic_waves", 0)


@pytest.mark.parametrize("waves", [0, 1])
@pytest.mark.parametrize("fused", [0, 1])
def test_generic_relpos_wave_split(gpu, waves, fused):
    """The tiny fp32 rel-pos config (8x8 grid, head_dim 16) on both wave modes,
    with the terms formed in the kernel and read from the workspace."""
    wl = workloads.WORKLOADS["tiny_relpos_fp32"]
    x = workloads.generate(wl, seed=3)
    g = {k_: t.cuda() for k_, t in x.items()}
    gpu.set_tuning("generic_waves", waves)
    gpu.set_tuning("relpos_fused", fused)
    try:
        o, lse = gpu.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=wl.layout,
                                 scale=wl.scale, return_lse=True)
        torch.cuda.synchronize()
        assert gpu.last_kernel() == "generic_fwd_kernel"
    finally:
        gpu.set_tuning("generic_waves", 0)
        gpu.set_tuning("relpos_fused", 1)
    rp = {"rel_pos_h": np64(x["rel_pos_h"]), "rel_pos_w": np64(x["rel_pos_w"]), "grid": wl.grid}
    ref = oracle.sdpa(np64(x["q"]), np64(x["k"]), np64(x["v"]), layout=wl.layout, scale=wl.scale, rel_pos=rp)
    assert max_err(np64(o), ref["o"]) <= TOL["fp32"]
    assert max_err(np64(lse), ref["lse"]) <= TOL["fp32"]


TERMS_GRIDS = [(14, 14), (64, 64), (40, 24), (5, 27), (16, 64), (9, 96), (3, 100), (8, 32), (4, 32)]


@pytest.mark.parametrize("mfma", [1, 0])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("grid", TERMS_GRIDS, ids=[f"{a}x{b}" for a, b in TERMS_GRIDS])
def test_relpos_terms_kernels(gpu, mfma, dtype, D, grid):
    """relpos_terms on the matrix cores (32-token blocks, products over the
    table rows each block needs, skewed read-out through LDS) and on the
    vector ALUs, against the oracle: grids whose 32-token blocks stay in one
    grid row (64 and 96 wide) or span several (14, 24, 27 wide), a ragged last
    block (5 x 27 = 135 tokens), head_dim 32 / 64 / 128, both layouts, a
    100-wide grid that only the vector kernel takes, and term rows of 4, 8,
    16, 32 and 64 floats (widths that divide a 256-float store step take the
    unrolled read-out)."""
    gh, gw = grid
    T, B, H = gh * gw, 2, 3
    layout = "bshd" if (gh + D) % 2 else "bhsd"
    q = rnd(layout_shape(B, H, T, D, layout), dtype, 60 + gh)
    g = torch.Generator().manual_seed(61 + gw)
    rh = (0.02 * torch.randn((2 * gh - 1, D), generator=g)).to(dtype)
    rw = (0.02 * torch.randn((2 * gw - 1, D), generator=g)).to(dtype)
    gpu.set_tuning("relpos_mfma", mfma)
    try:
        th, tw = gpu.relpos_terms(q.cuda(), rh.cuda(), rw.cuda(), grid, layout=layout)
        torch.cuda.synchronize()
    finally:
        gpu.set_tuning("relpos_mfma", 1)
    rth, rtw = oracle.relpos_terms(oracle.to_bhsd(np64(q), layout), np64(rh), np64(rw), gh, gw)
    assert max_err(np64(th), rth) <= 1e-4 and max_err(np64(tw), rtw) <= 1e-4


def test_relpos_terms_full_size(gpu):
    """SAM ViT-B global grid at full size (12 heads, 64 x 64, head_dim 64):
    both term arrays against the oracle, every element."""
    wl = workloads.WORKLOADS["sam_global_relpos"]
    x = workloads.generate(wl, seed=4)
    g = {k_: t.cuda() for k_, t in x.items()}
    th, tw = gpu.relpos_terms(g["q"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=wl.layout)
    torch.cuda.synchronize()
    rth, rtw = oracle.relpos_terms(oracle.to_bhsd(np64(x["q"]), wl.layout), np64(x["rel_pos_h"]),
                                   np64(x["rel_pos_w"]), *wl.grid)
    assert max_err(np64(th), rth) <= 1e-4 and max_err(np64(tw), rtw) <= 1e-4
