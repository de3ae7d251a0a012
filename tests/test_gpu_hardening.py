"""GPU hardening: guard bands around every buffer a kernel writes, bitwise
determinism of the headline and split-KV routes, and SAM ViT-B global
rel-pos attention at batch 4 (more query blocks than one round of
workgroups) in bf16 and fp16.

Guard bands: O, lse and the workspace are views into one device arena whose
bytes before and after each buffer are filled with NaN; the call goes
through the C ABI with those pointers, and afterwards every guard byte must
be unchanged and O must match the oracle.  A kernel that stores past the end
(or before the start) of a buffer fails here instead of corrupting a
neighbouring allocation unnoticed.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import TOL, gpu_inputs, max_err, np64, oracle_kwargs, rows_of, run_gpu, sample_picks

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of NaN before and after each written buffer
DT = {"fp32": 0, "bf16": 1, "fp16": 2}
LAY = {"bshd": 0, "bhsd": 1}


class Arena:
    """One NaN-filled device buffer holding several guarded regions."""

    def __init__(self, sizes):
        self.offs, tot = [], 0
        for n in sizes:
            tot += GUARD
            self.offs.append(tot)
            tot += (n + 255) // 256 * 256
        tot += GUARD
        self.buf = torch.full((tot // 4,), float("nan"), dtype=torch.float32, device="cuda")
        self.sizes = sizes
        self.snapshot = self.buf.clone()

    def ptr(self, i):
        return ctypes.c_void_p(self.buf.data_ptr() + self.offs[i]) if self.sizes[i] else None

    def view(self, i, dtype, shape):
        b = self.buf.view(torch.uint8)[self.offs[i]:self.offs[i] + self.sizes[i]]
        return b.view(dtype).view(shape)

    def guards_intact(self):
        """Every byte outside the regions still holds the initial NaN pattern."""
        keep = torch.ones(self.buf.numel() * 4, dtype=torch.bool, device="cuda")
        for o, n in zip(self.offs, self.sizes):
            keep[o:o + n] = False
        a = self.buf.view(torch.uint8)[keep]
        b = self.snapshot.view(torch.uint8)[keep]
        return bool(torch.equal(a, b))


CANARY_CASES = [
    # name, workload, layout, out fp32, tuning
    ("split64w_relpos_fused", "sam_global_relpos", "bhsd", True, {"split_wide": 2}),
    ("split64w_relpos_terms", "sam_global_relpos", "bshd", False, {"split_wide": 2, "relpos_fused": 0}),
    ("window", "sam_window_relpos", "bhsd", False, {}),
    ("d16_qpack_splitkv", "sam_decoder_q7", "bhsd", True, {"num_splits": 5}),
    ("d16_kpack", "sam_decoder_kv7", "bshd", False, {}),
    ("tiled_causal", "gqa_causal", "bshd", False, {}),
    ("tiled_splitkv", "gqa_decode", "bhsd", True, {}),
    ("generic_fp32_relpos", "tiny_relpos_fp32", "bhsd", True, {}),
    ("generic_relpos_terms", "tiny_relpos_fp32", "bshd", True, {"relpos_fused": 0}),
]


@pytest.mark.parametrize("case", CANARY_CASES, ids=[c[0] for c in CANARY_CASES])
def test_guard_bands_untouched(gpu, case):
    name, wname, layout, out32, tuning = case
    wl = workloads.replica(wname)
    print(f"[canary] {name} {wl}", flush=True)
    x = workloads.generate(wl, seed=2, layout=layout)
    g = gpu_inputs(x)
    lib = gpu.load()
    dt = DT[wl.dtype]
    odt = 0 if out32 else dt
    es_o = 4 if odt == 0 else (2 if dt else 4)
    try:
        for k, v in tuning.items():
            gpu.set_tuning(k, v)
        if wl.relpos:
            ws_n = lib.sdpa_workspace_size(dt, wl.B, wl.Hq, wl.Hkv, wl.Tq, wl.Tkv, wl.D, wl.scale, 1, *wl.grid)
        else:
            ws_n = lib.sdpa_workspace_size(dt, wl.B, wl.Hq, wl.Hkv, wl.Tq, wl.Tkv, wl.D, wl.scale, 0, 0, 0)
        if tuning.get("relpos_fused") == 0 or tuning.get("num_splits", 1) > 1 or wname == "gqa_decode":
            assert ws_n > 0            # the guarded workspace is really used
        n_o = g["q"].numel() * es_o
        n_l = wl.B * wl.Hq * wl.Tq * 4
        ar = Arena([n_o, n_l, ws_n])
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if wl.relpos:
            st = lib.sdpa_relpos_fwd(gpu._ptr(g["q"]), gpu._ptr(g["k"]), gpu._ptr(g["v"]), ar.ptr(0), dt, odt,
                                     LAY[layout], wl.B, wl.Hq, wl.grid[0], wl.grid[1], wl.D,
                                     gpu._ptr(g["rel_pos_h"]), gpu._ptr(g["rel_pos_w"]), wl.scale, ar.ptr(1),
                                     ar.ptr(2), ws_n, s)
        else:
            ms = gpu._mask_struct(wl.mask, wl.B, wl.Hq, wl.Tq, wl.Tkv, [], g["q"].device)
            st = lib.sdpa_fwd(gpu._ptr(g["q"]), gpu._ptr(g["k"]), gpu._ptr(g["v"]), ar.ptr(0), dt, odt, LAY[layout],
                              wl.B, wl.Hq, wl.Hkv, wl.Tq, wl.Tkv, wl.D, wl.scale, ctypes.byref(ms), ar.ptr(1),
                              ar.ptr(2), ws_n, s)
        assert st == 0, lib.sdpa_last_error()
        torch.cuda.synchronize()
    finally:
        gpu.set_tuning("split_wide", 1)
        gpu.set_tuning("relpos_fused", 1)
        gpu.set_tuning("num_splits", 0)
    assert ar.guards_intact(), f"{name}: a kernel wrote outside O, lse or the workspace"
    o = ar.view(0, torch.float32 if odt == 0 else g["q"].dtype, tuple(g["q"].shape))
    lse = ar.view(1, torch.float32, (wl.B, wl.Hq, wl.Tq))
    ref = oracle.sdpa(np64(x["q"]), np64(x["k"]), np64(x["v"]), **oracle_kwargs(wl, x, layout))
    tol = TOL[wl.dtype] + (0.0 if odt == 0 else float(np.abs(ref["o"]).max()) * 2.0 ** -8)
    assert max_err(np64(o), ref["o"]) <= tol
    assert max_err(np64(lse), ref["lse"]) <= TOL[wl.dtype]


@pytest.mark.parametrize("name", ["sam_global_relpos", "sam_decoder_q7", "gqa_decode"])
def test_bitwise_determinism_full_size(gpu, name):
    """The headline kernel (12-wave workgroups, terms formed in the kernel) and
    both split-KV routes (head_dim 16 and 128; partials merged in a fixed
    order) at full size: two
    calls on the same inputs give the same bits, output and lse."""
    wl = workloads.WORKLOADS[name]
    x = workloads.generate(wl, seed=0)
    g = gpu_inputs(x)
    a = run_gpu(gpu, wl, g, wl.layout, out_dtype=None, return_lse=True)
    k1 = gpu.last_kernel()
    b = run_gpu(gpu, wl, g, wl.layout, out_dtype=None, return_lse=True)
    torch.cuda.synchronize()
    assert k1 == {"sam_global_relpos": "flash_split64w_kernel", "sam_decoder_q7": "d16_qpack_kernel",
                  "gqa_decode": "flash_tiled_kernel"}[name]
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.slow
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_sam_global_batch4_sampled_rows(gpu, dtype):
    """SAM ViT-B global rel-pos attention at batch 4: 6144 query blocks, i.e.
    four rounds of the 12-wave workgroups; sampled rows of every batch entry
    against the oracle, on the matrix-core route with the terms formed in the
    kernel."""
    wl = workloads.WORKLOADS["sam_global_relpos"].with_(B=4, dtype=dtype)
    x = workloads.generate(wl, seed=5)
    g = gpu_inputs(x)
    o, lse = run_gpu(gpu, wl, g, wl.layout, return_lse=True)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == "flash_split64w_kernel"
    assert gpu.relpos_fused(g["q"].dtype, wl.D, wl.grid)
    picks = sample_picks(wl, n_random=40, seed=5)
    picks += [(b, h, i) for b in range(4) for (h, i) in ((3, 100), (11, 4095), (6, 2048))]
    ro, rl = oracle.sdpa_rows(np64(x["q"]), np64(x["k"]), np64(x["v"]), picks, **oracle_kwargs(wl, x, wl.layout))
    assert max_err(np64(rows_of(o, picks, wl.layout)), ro) <= TOL[dtype]
    assert max_err(np64(torch.stack([lse[b, h, i] for b, h, i in picks])), rl) <= TOL[dtype]
    assert torch.isfinite(o).all()
