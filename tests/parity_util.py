"""Shared helpers for the GPU parity tests: run one workload through the HIP
library and through the oracle on the same seeded inputs."""
import numpy as np
import torch

import oracle
import workloads

# Max-abs tolerances on unit-variance data with fp32 accumulation: 1e-4 for
# fp32 inputs, 1.5e-2 for bf16 inputs, 5e-3 for fp16 inputs (the probabilities
# are rounded to the input type before P.V: 2^-9 relative for bf16, 2^-11 for
# fp16, times a few units of |v|).  A bf16 OUTPUT additionally carries its
# own rounding (half an ulp, |O| * 2^-9), added to the bound when checked.
TOL = {"fp32": 1e-4, "bf16": 1.5e-2, "fp16": 5e-3}


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_inputs(x):
    return {k: v.cuda() for k, v in x.items()}


def oracle_kwargs(wl, x, layout):
    kw = {"layout": layout, "scale": wl.scale, "mask": wl.mask}
    if wl.relpos:
        kw["rel_pos"] = {"rel_pos_h": np64(x["rel_pos_h"]), "rel_pos_w": np64(x["rel_pos_w"]), "grid": wl.grid}
    return kw


def run_gpu(fa, wl, g, layout, out_dtype=torch.float32, return_lse=False):
    if wl.relpos:
        return fa.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=layout,
                              scale=wl.scale, out_dtype=out_dtype, return_lse=return_lse)
    return fa.sdpa(g["q"], g["k"], g["v"], layout=layout, scale=wl.scale, mask=wl.mask, out_dtype=out_dtype,
                   return_lse=return_lse)


def run_oracle(wl, x, layout):
    return oracle.sdpa(np64(x["q"]), np64(x["k"]), np64(x["v"]), **oracle_kwargs(wl, x, layout))


def sample_picks(wl, n_random=48, seed=0):
    """Rows checked at full size: the first and last rows of a few heads plus random ones."""
    rng = np.random.default_rng(seed)
    picks = set()
    for b in {0, wl.B - 1}:
        for h in {0, wl.Hq - 1}:
            for i in (0, 1, 31, 32, 63, 64, wl.Tq - 1, wl.Tq // 2):
                if 0 <= i < wl.Tq:
                    picks.add((b, h, i))
    for _ in range(n_random):
        picks.add((int(rng.integers(wl.B)), int(rng.integers(wl.Hq)), int(rng.integers(wl.Tq))))
    return sorted(picks)


def rows_of(o, picks, layout):
    out = []
    for b, h, i in picks:
        out.append(o[b, h, i] if layout == "bhsd" else o[b, i, h])
    return torch.stack(out)


def max_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite GPU output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0
