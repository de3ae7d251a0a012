"""GPU parity: the HIP library against the fp64 oracle on the same seeded
inputs -- small replicas of every workload element by element (both layouts),
every workload at full size on sampled rows, and edge cases."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import (TOL, gpu_inputs, max_err, np64, oracle_kwargs, rows_of, run_gpu, run_oracle,
                         sample_picks)

pytestmark = pytest.mark.gpu
NAMES = list(workloads.WORKLOADS)


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("name", NAMES)
def test_replica_elementwise(gpu, name, layout):
    wl = workloads.replica(name)
    print(f"[parity] replica {name} {layout} {wl}", flush=True)
    x = workloads.generate(wl, seed=0, layout=layout)
    o, lse = run_gpu(gpu, wl, gpu_inputs(x), layout, return_lse=True)
    torch.cuda.synchronize()
    ref = run_oracle(wl, x, layout)
    err = max_err(np64(o), ref["o"])
    assert err <= TOL[wl.dtype], f"{name} {layout}: max-abs {err:.3e}"
    lerr = max_err(np64(lse), ref["lse"])
    assert lerr <= TOL[wl.dtype], f"{name} {layout}: lse max-abs {lerr:.3e}"
    # bf16 output: the same bound plus the output's own rounding
    ob = run_gpu(gpu, wl, gpu_inputs(x), layout, out_dtype=None)
    d = np.abs(np64(ob) - ref["o"]) - np.abs(ref["o"]) * 2.0 ** -9
    assert d.max() <= TOL[wl.dtype], f"{name} {layout}: output-dtype excess {d.max():.3e}"


@pytest.mark.parametrize("name", NAMES)
def test_full_size_sampled_rows(gpu, name):
    wl = workloads.WORKLOADS[name]
    print(f"[parity] full {name}", flush=True)
    x = workloads.generate(wl, seed=0)
    g = gpu_inputs(x)
    o, lse = run_gpu(gpu, wl, g, wl.layout, return_lse=True)
    torch.cuda.synchronize()
    picks = sample_picks(wl)
    ro, rl = oracle.sdpa_rows(np64(x["q"]), np64(x["k"]), np64(x["v"]), picks, **oracle_kwargs(wl, x, wl.layout))
    err = max_err(np64(rows_of(o, picks, wl.layout)), ro)
    assert err <= TOL[wl.dtype], f"{name}: sampled max-abs {err:.3e}"
    lsel = torch.stack([lse[b, h, i] for b, h, i in picks])
    assert max_err(np64(lsel), rl) <= TOL[wl.dtype]
    assert torch.isfinite(o).all()


F16_NAMES = [n for n in NAMES if workloads.WORKLOADS[n].dtype == "bf16"]


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
@pytest.mark.parametrize("name", F16_NAMES)
def test_replica_fp16(gpu, name, layout):
    """fp16 inputs on every 16-bit route: the same kernel as bf16, within the
    fp16 bound (probabilities rounded to fp16), lse, and fp16 output."""
    wb = workloads.replica(name)
    run_gpu(gpu, wb, gpu_inputs(workloads.generate(wb, seed=1, layout=layout)), layout)
    torch.cuda.synchronize()
    kernel_bf16 = gpu.last_kernel()
    wl = workloads.replica(name, dtype="fp16")
    print(f"[parity] fp16 replica {name} {layout}", flush=True)
    x = workloads.generate(wl, seed=1, layout=layout)
    o, lse = run_gpu(gpu, wl, gpu_inputs(x), layout, return_lse=True)
    torch.cuda.synchronize()
    assert gpu.last_kernel() == kernel_bf16
    ref = run_oracle(wl, x, layout)
    err = max_err(np64(o), ref["o"])
    assert err <= TOL["fp16"], f"{name} {layout}: max-abs {err:.3e}"
    assert max_err(np64(lse), ref["lse"]) <= TOL["fp16"]
    ob = run_gpu(gpu, wl, gpu_inputs(x), layout, out_dtype=None)
    assert ob.dtype == torch.float16
    d = np.abs(np64(ob) - ref["o"]) - np.abs(ref["o"]) * 2.0 ** -11
    assert d.max() <= TOL["fp16"], f"{name} {layout}: output-dtype excess {d.max():.3e}"


def test_full_size_fp16_global_relpos(gpu):
    wl = workloads.WORKLOADS["sam_global_relpos"].with_(dtype="fp16")
    x = workloads.generate(wl, seed=0)
    o, lse = run_gpu(gpu, wl, gpu_inputs(x), wl.layout, return_lse=True)
    torch.cuda.synchronize()
    picks = sample_picks(wl, n_random=24)
    ro, rl = oracle.sdpa_rows(np64(x["q"]), np64(x["k"]), np64(x["v"]), picks, **oracle_kwargs(wl, x, wl.layout))
    assert max_err(np64(rows_of(o, picks, wl.layout)), ro) <= TOL["fp16"]
    assert max_err(np64(torch.stack([lse[b, h, i] for b, h, i in picks])), rl) <= TOL["fp16"]


def test_relpos_terms_match_oracle(gpu):
    for name in ("tiny_relpos_fp32", "sam_window_relpos", "sam_global_relpos"):
        wl = workloads.replica(name)
        for layout in ("bhsd", "bshd"):
            x = workloads.generate(wl, seed=3, layout=layout)
            g = gpu_inputs(x)
            th, tw = gpu.relpos_terms(g["q"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=layout)
            rth, rtw = oracle.relpos_terms(oracle.to_bhsd(np64(x["q"]), layout), np64(x["rel_pos_h"]),
                                           np64(x["rel_pos_w"]), *wl.grid)
            tol = 1e-5 if wl.dtype == "fp32" else 1e-4
            assert max_err(np64(th), rth) <= tol and max_err(np64(tw), rtw) <= tol, (name, layout)
