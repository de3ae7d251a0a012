"""The allocation-free forward entry point (sdpa_fwd_noalloc) against sdpa_fwd,
called directly through the C ABI: two calls in a row, the second smaller, on
the split-KV route whose partials live in the library's fixed device scratch,
plus a route with no scratch at all.  Kept last in collection order."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, max_err, np64

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Tq, Tkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda H, T: torch.randn((B, H, T, D), generator=g).to(torch.bfloat16).cuda()
    return mk(Hq, Tq), mk(Hkv, Tkv), mk(Hkv, Tkv)


def _abi_noalloc(fa, q, k, v, o, lse, scale, mask=None):
    lib = fa.load()
    B, Hq, Tq, D = q.shape
    Hkv, Tkv = k.shape[1], k.shape[2]
    ms = fa._mask_struct(mask, B, Hq, Tq, Tkv, [], q.device)
    st = lib.sdpa_fwd_noalloc(fa._ptr(q), fa._ptr(k), fa._ptr(v), fa._ptr(o), 1, 0, 1, B, Hq, Hkv, Tq, Tkv, D,
                              scale, ctypes.byref(ms), fa._ptr(lse),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.sdpa_last_error()


@pytest.mark.parametrize("shapes", [
    # SAM mask-decoder shape (7 tokens x 4096 keys, head_dim 16: split-KV), then a smaller one
    [(1, 8, 8, 7, 4096, 16), (1, 4, 2, 3, 1000, 16)],
    # no scratch needed (head_dim 64): the entry point runs the same kernels with no partials
    [(2, 4, 2, 100, 300, 64), (1, 2, 1, 40, 50, 64)],
    # head_dim 128 / 64 decode shapes: split-KV on the double-buffered kernel, partials in the scratch
    [(1, 32, 8, 1, 8192, 128), (1, 8, 8, 4, 2048, 64)],
])
def test_noalloc_matches_sdpa_fwd(gpu, shapes):
    lib = gpu.load()
    for i, (B, Hq, Hkv, Tq, Tkv, D) in enumerate(shapes):
        print(f"[noalloc] call {i}: B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tkv{Tkv} D{D}", flush=True)
        q, k, v = _inputs(B, Hq, Hkv, Tq, Tkv, D, seed=10 + i)
        scale = 1.0 / np.sqrt(D)
        ws_n = lib.sdpa_workspace_size(1, B, Hq, Hkv, Tq, Tkv, D, scale, 0, 0, 0)
        if (D == 16 and Tq <= 8) or (Tq <= 4 and Tkv >= 2048):
            assert ws_n > 0                       # this call really uses the split-KV scratch
        ref, ref_lse = gpu.sdpa(q, k, v, scale=scale, out_dtype=torch.float32, return_lse=True)
        o = torch.full((B, Hq, Tq, D), float("nan"), device="cuda")
        lse = torch.full((B, Hq, Tq), float("nan"), device="cuda")
        _abi_noalloc(gpu, q, k, v, o, lse, scale)
        torch.cuda.synchronize()
        assert gpu.last_kernel() in ("d16_qpack_kernel", "flash_tiled_kernel", "flash_split64_kernel",
                                     "flash_split64w_kernel")
        # the same kernels on the same inputs: the partials live elsewhere, the arithmetic is identical
        assert torch.equal(o, ref), float((o - ref).abs().max())
        assert torch.equal(lse, ref_lse)
        # and within the parity bound of the fp64 oracle
        want = oracle.sdpa(np64(q), np64(k), np64(v), scale=scale)
        assert max_err(np64(o), want["o"]) <= TOL["bf16"]
        assert max_err(np64(lse), want["lse"]) <= TOL["bf16"]


def test_noalloc_rejects_oversized_scratch(gpu):
    """A forced split count whose partials exceed the fixed scratch is refused before any launch."""
    lib = gpu.load()
    q, k, v = _inputs(1, 64, 64, 8, 65536, 16, seed=3)
    o = torch.empty((1, 64, 8, 16), device="cuda")
    gpu.set_tuning("num_splits", 1024)
    try:
        ms = gpu._mask_struct(None, 1, 64, 8, 65536, [], q.device)
        st = lib.sdpa_fwd_noalloc(gpu._ptr(q), gpu._ptr(k), gpu._ptr(v), gpu._ptr(o), 1, 0, 1, 1, 64, 64, 8, 65536,
                                  16, 0.25, ctypes.byref(ms), None, None)
        msg = lib.sdpa_last_error()
    finally:
        gpu.set_tuning("num_splits", 0)
    assert st == -2 and b"scratch" in msg


def test_noalloc_lowers_an_automatic_split_count(gpu):
    """A head_dim-128 shape whose automatic split-KV partials (16 chunks, 33 MB)
    exceed the fixed 8 MiB scratch: the entry point runs with fewer chunks
    instead of failing, and the result stays within the parity bound of
    sdpa_fwd's 16-chunk result and of the oracle (sampled rows)."""
    lib = gpu.load()
    B, Hq, Hkv, Tq, Tkv, D = 1, 16, 16, 256, 8192, 128
    print(f"[noalloc] capped split: B{B} Hq{Hq} Tq{Tq} Tkv{Tkv} D{D}", flush=True)
    assert lib.sdpa_workspace_size(1, B, Hq, Hkv, Tq, Tkv, D, float("nan"), 0, 0, 0) > (8 << 20)
    q, k, v = _inputs(B, Hq, Hkv, Tq, Tkv, D, seed=30)
    scale = 1.0 / np.sqrt(D)
    ref, ref_lse = gpu.sdpa(q, k, v, scale=scale, out_dtype=torch.float32, return_lse=True)
    for _ in range(2):
        o = torch.full((B, Hq, Tq, D), float("nan"), device="cuda")
        lse = torch.full((B, Hq, Tq), float("nan"), device="cuda")
        _abi_noalloc(gpu, q, k, v, o, lse, scale)
        torch.cuda.synchronize()
        assert gpu.last_kernel() == "flash_tiled_kernel"
        assert max_err(np64(o), np64(ref)) <= TOL["bf16"]
        assert max_err(np64(lse), np64(ref_lse)) <= TOL["bf16"]
    rows = [(h, i) for h in (0, 7, 15) for i in (0, 1, 100, 255)]
    qs = torch.stack([q[0, h, i] for h, i in rows]).view(1, len(rows), 1, D)
    ks = torch.stack([k[0, h] for h, _ in rows]).unsqueeze(0)
    vs = torch.stack([v[0, h] for h, _ in rows]).unsqueeze(0)
    want = oracle.sdpa(np64(qs), np64(ks), np64(vs), scale=scale)
    got = torch.stack([o[0, h, i] for h, i in rows]).view(1, len(rows), 1, D)
    assert max_err(np64(got), want["o"]) <= TOL["bf16"]
