"""Benchmark: attention TFLOP/s (and % of MI355X dense bf16 MFMA peak) of the
fused rel-pos SDPA on SAM ViT-B's 64x64 global attention (B1, 12 heads,
T 4096, head_dim 64, bf16), one sdpa_relpos_fwd call per step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --copy-calibration MIB [--steps K]


Prints ONE JSON line.  A step is one full pass of the fused path (rel-pos
terms + flash attention, all on the GPU) over the seeded synthetic inputs,
which are resident in HBM before timing starts.  `roofline` describes the
dominant kernel (the flash attention kernel); `cpu_baseline` times the fp64
CPU oracle on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, published

# Source file of each attention kernel, for matching recorded counter data.
KERNEL_SOURCE = {
    "flash_split64_kernel": "flash_split64.hip",
    "flash_split64w_kernel": "flash_split64w.hip",
    "flash_tiled_kernel": "flash_tiled.hip",
    "flash_window_kernel": "flash_window.hip",
    "flash_mfma_kernel": "flash_mfma.hip",
    "d16_qpack_kernel": "flash_d16.hip",
    "d16_kpack_kernel": "flash_d16.hip",
    "generic_fwd_kernel": "generic_fwd.hip",
}


def allowed_pairs(wl):
    """Number of (query, key) pairs the mask allows, per (batch, head)."""
    Tq, Tkv = wl.Tq, wl.Tkv
    if wl.mask is None:
        return Tq * Tkv
    d = wl.mask.get("offset", 0)
    tot = 0
    for i in range(Tq):
        hi = min(Tkv - 1, i + d)
        lo = 0 if wl.mask["kind"] == "causal" else max(0, i + d - wl.mask["window"] + 1)
        tot += max(0, hi - lo + 1)
    return tot


def flop_model(wl):
    """Algorithmic FLOPs: 4*D per allowed pair (Q.K^T and P.V), plus for rel-pos
    2*D per term entry (B*H*T*(grid_h+grid_w) dot products) and 2 adds per score."""
    pairs = allowed_pairs(wl) * wl.B * wl.Hq
    attn = 4 * wl.D * pairs
    bias = 0
    if wl.relpos:
        gh, gw = wl.grid
        bias = 2 * wl.B * wl.Hq * wl.Tq * (gh + gw) * wl.D + 2 * pairs
    return attn, bias


def byte_model(wl):
    """Algorithmic HBM bytes of one call: read Q, K, V once, write O once."""
    es = 4 if wl.dtype == "fp32" else 2
    return es * wl.D * (2 * wl.B * wl.Hq * wl.Tq + 2 * wl.B * wl.Hkv * wl.Tkv)


def run_call(fa, wl, g, out):
    if "bias" in g:                 # the materialised-bias route: rel-pos bias as an additive mask
        return fa.sdpa(g["q"], g["k"], g["v"], layout=wl.layout, scale=wl.scale,
                       mask={"kind": "additive", "data": g["bias"]}, out=out)
    if wl.relpos:
        return fa.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=wl.layout,
                              scale=wl.scale, out=out, workspace=g.get("ws"))
    return fa.sdpa(g["q"], g["k"], g["v"], layout=wl.layout, scale=wl.scale, mask=wl.mask, out=out)


MALL_BYTES = 256 * 2**20            # MI355X Infinity Cache: working sets below this can stay cache-resident
ROTATE_BYTES = 512 * 2**20          # span of distinct buffer sets that HBM-cold timing cycles through


def buffer_sets(g, min_bytes=ROTATE_BYTES):
    """Distinct copies of the call's inputs and output, laid out one after the
    other in one device arena spanning at least `min_bytes`, so that cycling
    through them reads every input from HBM rather than from the caches.
    Working sets of MALL size or more need no copies: one set is returned.
    Each set is a dict like `g` plus its own "out"."""
    import torch
    names = [k for k in ("q", "k", "v", "rel_pos_h", "rel_pos_w", "bias", "ws") if k in g]
    al = lambda n: (n + 255) // 256 * 256
    offs, sb = {}, 0
    for k in names + ["out"]:
        t = g["q"] if k == "out" else g[k]
        offs[k] = sb
        sb += al(t.numel() * t.element_size())
    if sb >= MALL_BYTES:
        one = dict(g)
        one["out"] = torch.empty_like(g["q"])
        return [one]
    nsets = (min_bytes + sb - 1) // sb
    arena = torch.empty(nsets * sb, dtype=torch.uint8, device=g["q"].device)
    tmpl = torch.zeros(sb, dtype=torch.uint8, device=g["q"].device)
    for k in names:
        n = g[k].numel() * g[k].element_size()
        tmpl[offs[k]:offs[k] + n].copy_(g[k].contiguous().view(-1).view(torch.uint8))
    arena.view(nsets, sb).copy_(tmpl.expand(nsets, sb))
    sets = []
    for i in range(nsets):
        d = {}
        for k in names + ["out"]:
            t = g["q"] if k == "out" else g[k]
            n = t.numel() * t.element_size()
            d[k] = arena[i * sb + offs[k]:i * sb + offs[k] + n].view(t.dtype).view(t.shape)
        sets.append(d)
    return sets


def time_gpu(fa, wl, sets, steps, warmup):
    """Host-clocked seconds per call over `steps` calls (synchronised on both
    sides), cycling through the buffer sets."""
    import torch
    for i in range(warmup):
        run_call(fa, wl, sets[i % len(sets)], sets[i % len(sets)]["out"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        s = sets[i % len(sets)]
        run_call(fa, wl, s, s["out"])
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def _hold_stream(ms):
    """Keep the current stream busy for about `ms` milliseconds (a bounded
    spin kernel), so that the launches queued behind it run back to back and
    HIP events between them time the GPU work, not the host's launch rate."""
    import torch
    global _SPIN_PER_MS
    if _SPIN_PER_MS is None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        torch.cuda._sleep(1_000_000)
        ev[1].record()
        ev[1].synchronize()
        _SPIN_PER_MS = 1_000_000 / max(ev[0].elapsed_time(ev[1]), 1e-3)
    torch.cuda._sleep(int(min(ms, 200.0) * _SPIN_PER_MS))


_SPIN_PER_MS = None


def kernel_events(fa, wl, sets, steps, reps=5):
    """GPU duration per call of the whole call and of the separate rel-pos terms
    launch, from HIP events recorded on the stream the kernels run on (torch's
    current stream, which the binding passes to the library).  The launches of
    each repetition queue up behind a spin kernel, so they run back to back,
    cycling through the buffer sets.  Returns the median and the min over
    `reps` repetitions of (call ms, terms ms)."""
    import statistics
    import torch
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            _hold_stream(2.0 + 0.2 * steps)
            ev[0].record(s)
            for i in range(steps):
                fn(sets[i % len(sets)])
            ev[1].record(s)
            ev[1].synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) / steps)
        return statistics.median(ts), min(ts)

    call_med, call_min = timed(lambda b: run_call(fa, wl, b, b["out"]))
    terms_med = terms_min = 0.0
    g = sets[0]
    if wl.relpos and "bias" not in g and not fa.relpos_fused(g["q"].dtype, wl.D, wl.grid):
        terms_med, terms_min = timed(lambda b: fa.relpos_terms(b["q"], b["rel_pos_h"], b["rel_pos_w"], wl.grid,
                                                                layout=wl.layout))
    return (call_med, call_min), (terms_med, terms_min)


def source_sha256(kernel):
    import hashlib
    path = os.path.join(ROOT, "attention_flash_sdpa_amd", "csrc", KERNEL_SOURCE.get(kernel, ""))
    if not os.path.isfile(path):
        return None
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the recorded FETCH_SIZE / WRITE_SIZE counter
    runs (scaled by the plain-copy calibration), if a record exists for this
    kernel and workload AND was taken on the kernel source as it is now."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.isfile(path):
        return None, "no counter record"
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic: "):
                rec = json.loads(line[len("traffic: "):])
                break
    if rec is None:
        return None, "counter record has no traffic line"
    if rec.get("source_sha256") != source_sha256(kernel):
        return None, "counters predate the current kernel source"
    return rec["bytes_per_launch"], f"{os.path.relpath(path, ROOT)}"


def copy_calibration(mib, steps):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    per dispatch calibrate the counters against true bytes."""
    import torch
    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": n, "read_bytes": n, "write_bytes": n, "steps": steps}))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, budget_s=20.0):
    """Time the fp64 oracle on whole heads (every batch entry) of the same inputs
    until about `budget_s` seconds of CPU work are done; report it at the
    metric's unit."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    f64 = lambda t: t.to("cpu").double().numpy()
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    kw = {"layout": wl.layout, "scale": wl.scale, "mask": wl.mask}
    if wl.relpos:
        kw["rel_pos"] = {"rel_pos_h": f64(x["rel_pos_h"]), "rel_pos_w": f64(x["rel_pos_w"]), "grid": wl.grid}
    hsel = lambda a, h, grp=1: (a[:, h // grp:h // grp + 1] if wl.layout == "bhsd" else a[:, :, h // grp:h // grp + 1])
    grp = wl.Hq // wl.Hkv
    done, t_total = 0, 0.0
    for h in range(wl.Hq):
        t0 = time.perf_counter()
        oracle.sdpa(hsel(q, h), hsel(k, h, grp), hsel(v, h, grp), **kw)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    sub = wl.with_(Hq=done, Hkv=max(1, done // grp))
    attn, bias = flop_model(sub)
    frac = done / wl.Hq
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return {"value": round((attn + bias) / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} of {wl.Hq} heads (each over all {wl.B} batch entries; {frac:.3f} of the "
                      f"workload), fp64 numpy, {t_total:.1f} s wall"}


def bench_backward(fa, wl, x, g, args):
    """One backward call per step (sdpa_backward, or sdpa_relpos_backward for rel-pos
    workloads): delta, dK/dV and dQ kernels (plus the rel-pos terms and tail).
    Algorithmic FLOPs are those of the five products per allowed pair
    (S = Q.K^T, dW = dO.V^T, dV, dK, dQ: 10 * D), the usual accounting of 2.5x
    the forward pass, plus the rel-pos products."""
    import statistics
    import numpy as np
    import torch
    rng = np.random.default_rng(1)
    do = torch.from_numpy(rng.standard_normal(tuple(x["q"].shape), dtype=np.float32)).to(g["q"].dtype).cuda()
    if wl.relpos:
        o, lse = fa.sdpa_relpos(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=wl.layout,
                                scale=wl.scale, return_lse=True)
        n = fa.load().sdpa_relpos_bwd_workspace_size(wl.B, wl.Hq, wl.grid[0], wl.grid[1], wl.D)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        call = lambda: fa.sdpa_relpos_backward(g["q"], g["k"], g["v"], o, do, lse, g["rel_pos_h"], g["rel_pos_w"],
                                               wl.grid, layout=wl.layout, scale=wl.scale, workspace=ws)
    else:
        o, lse = fa.sdpa(g["q"], g["k"], g["v"], layout=wl.layout, scale=wl.scale, mask=wl.mask, return_lse=True)
        call = lambda: fa.sdpa_backward(g["q"], g["k"], g["v"], o, do, lse, layout=wl.layout, scale=wl.scale,
                                        mask=wl.mask)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for _ in range(5):
        torch.cuda.synchronize()
        _hold_stream(2.0 + 1.5 * args.steps)
        ev[0].record(s)
        for _ in range(args.steps):
            call()
        ev[1].record(s)
        ev[1].synchronize()
        ts.append(ev[0].elapsed_time(ev[1]) / args.steps)
    call_ms = statistics.median(ts)
    pairs = allowed_pairs(wl) * wl.B * wl.Hq
    flops = 10 * wl.D * pairs
    if wl.relpos:       # terms recomputed, the tables' part of dQ, the tables' gradients: 2 D (gh + gw) per query each
        flops += 3 * 2 * wl.D * (wl.grid[0] + wl.grid[1]) * wl.B * wl.Hq * wl.Tq
    achieved = flops / (call_ms * 1e-3) / 1e12
    es = 2
    nbytes = es * wl.D * (4 * wl.B * wl.Hq * wl.Tq + 4 * wl.B * wl.Hkv * wl.Tkv) + 8 * wl.B * wl.Hq * wl.Tq
    line = {
        "metric": "attention backward TFLOP/s (10 D per allowed pair)",
        "value": round(flops / sec / 1e12, 3),
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100.0 * flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp16": "f16"}.get(wl.dtype, "f32"), "data": "synthetic",
        "config": {"workload": wl.name + "_backward", "description": wl.description + ", backward pass",
                   "layout": wl.layout, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "Tq": wl.Tq, "Tkv": wl.Tkv,
                   "head_dim": wl.D, "mask": wl.mask, "grid": list(wl.grid) if wl.grid else None,
                   "scale": wl.scale, "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "bwd_delta_kernel + bwd_dkdv_kernel + bwd_dq_kernel" +
                               (" + rel-pos terms and tail (one call)" if wl.relpos else " (one call)"),
                     "kernel_ms": round(call_ms, 5), "flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes},
    }
    print(json.dumps(line))


def _events_ms(call, steps, hold_ms):
    """Median over 5 repetitions of the HIP-event time per call, launches queued behind a spin."""
    import statistics
    import torch
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for _ in range(5):
        torch.cuda.synchronize()
        _hold_stream(hold_ms)
        ev[0].record(s)
        for _ in range(steps):
            call()
        ev[1].record(s)
        ev[1].synchronize()
        ts.append(ev[0].elapsed_time(ev[1]) / steps)
    return statistics.median(ts)


def bench_train_forward(fa, wl, g, args):
    """'dropout': per step, draw the keep bits (Philox4x32-10, one bit per score) and run the
    forward pass with attention dropout; the forward kernel's roofline is reported (attention
    FLOPs as for the forward pass), and the keep-bit kernel's time beside it.
    'weights': the [B, Hq, Tq, Tkv] fp32 attention weights rebuilt from lse (a debug output):
    bound by writing 4 bytes per score."""
    import torch
    if wl.relpos:
        print("bench.py: --pass dropout / weights take unmasked or index-masked workloads", file=sys.stderr)
        sys.exit(2)
    rate = 0.1
    pairs = allowed_pairs(wl) * wl.B * wl.Hq
    if args.pass_ == "dropout":
        keep = fa.dropout_mask(1, 0, rate, wl.B, wl.Hq, wl.Tq, wl.Tkv)
        out = torch.empty_like(g["q"])
        fwd = lambda: fa.sdpa(g["q"], g["k"], g["v"], layout=wl.layout, scale=wl.scale, mask=wl.mask, out=out,
                              dropout={"keep": keep, "rate": rate})
        mask_call = lambda: fa.dropout_mask(1, 0, rate, wl.B, wl.Hq, wl.Tq, wl.Tkv)
        step = lambda: (mask_call(), fwd())
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / args.steps
        fwd_ms = _events_ms(fwd, args.steps, 2.0 + 1.0 * args.steps)
        fwd()
        kernel = fa.last_kernel()
        mask_ms = _events_ms(mask_call, args.steps, 2.0 + 0.2 * args.steps)
        flops = 4 * wl.D * pairs
        achieved = flops / (fwd_ms * 1e-3) / 1e12
        keep_bytes = wl.B * wl.Hq * wl.Tq * ((wl.Tkv + 31) // 32) * 4
        line = {"metric": "attention TFLOP/s with attention dropout (keep bits drawn every step)",
                "value": round(flops / sec / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": {"bf16": "bf16", "fp16": "f16"}.get(wl.dtype, "f32"),
                "data": "synthetic",
                "config": {"workload": wl.name + "_dropout", "rate": rate, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv,
                           "Tq": wl.Tq, "Tkv": wl.Tkv, "head_dim": wl.D, "mask": wl.mask, "flop_per_step": flops},
                "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                             "kernel": kernel, "kernel_ms": round(fwd_ms, 5)},
                "keep_bits": {"kernel": "dropout_mask_kernel", "kernel_ms": round(mask_ms, 5), "bytes": keep_bytes,
                              "GB_per_s": round(keep_bytes / (mask_ms * 1e-3) / 1e9, 1)}}
    else:
        o, lse = fa.sdpa(g["q"], g["k"], g["v"], layout=wl.layout, scale=wl.scale, mask=wl.mask, return_lse=True)
        call = lambda: fa.attention_weights(g["q"], g["k"], lse, layout=wl.layout, scale=wl.scale, mask=wl.mask)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / args.steps
        ms = _events_ms(call, args.steps, 2.0 + 1.0 * args.steps)
        call()
        kernel = fa.last_kernel()
        elem = 2 if wl.dtype in ("bf16", "fp16") else 4
        wbytes = wl.B * wl.Hq * wl.Tq * wl.Tkv * 4
        # algorithmic bytes: the fp32 weights written once, Q, K and lse read once
        nbytes = wbytes + (wl.B * wl.Hq * wl.Tq + wl.B * wl.Hkv * wl.Tkv) * wl.D * elem + wl.B * wl.Hq * wl.Tq * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        # 2 D FLOPs per score: on the matrix cores (16-bit inputs) the write bounds the kernel; on the
        # vector ALUs (fp32 inputs, other head dims) whichever of the two takes longer at peak does
        vflops = 2 * wl.D * wl.B * wl.Hq * wl.Tq * wl.Tkv
        alu_bound = (kernel == "attn_weights_kernel"
                     and vflops / (FP32_VECTOR_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9))
        line = {"metric": "attention-weights output GB/s (fp32 [B, Hq, Tq, Tkv])",
                "value": round(nbytes / sec / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": {"bf16": "bf16", "fp16": "f16"}.get(wl.dtype, "f32"),
                "data": "synthetic",
                "config": {"workload": wl.name + "_weights", "B": wl.B, "Hq": wl.Hq, "Tq": wl.Tq, "Tkv": wl.Tkv,
                           "head_dim": wl.D, "mask": wl.mask},
                "roofline": ({"bound": "alu", "achieved": round(vflops / (ms * 1e-3) / 1e12, 3),
                              "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(vflops / (ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS, 4)}
                             if alu_bound else
                             {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(gbs / HBM_PEAK_GBS, 4)})}
        line["roofline"].update({"traffic": None, "kernel": kernel, "kernel_ms": round(ms, 5),
                                 "algorithmic_bytes_per_launch": nbytes, "flop_per_launch": vflops,
                                 "write_GB_per_s": round(wbytes / (ms * 1e-3) / 1e9, 1)})
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sam_global_relpos")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--dtype", choices=["bf16", "fp16"], default=None,
                    help="override the workload's 16-bit input type (fp16 runs the same kernels)")
    ap.add_argument("--route", choices=["relpos", "additive"], default="relpos",
                    help="rel-pos workloads: 'additive' times the bias materialised as a [B, H, T, T] "
                         "additive mask in the input dtype (formed before timing) instead of the fused terms")
    ap.add_argument("--pass", dest="pass_", choices=["forward", "backward", "dropout", "weights"], default="forward",
                    help="'backward' times one backward call per step (dQ, dK, dV from the forward pass's O and "
                         "lse, formed before timing); 'dropout' times drawing the keep bits plus the forward "
                         "pass with attention dropout (rate 0.1); 'weights' times the attention-weights output "
                         "(unmasked or index-masked workloads)")
    ap.add_argument("--head-dim", type=int, default=0, metavar="D",
                    help="override the workload's head_dim (16-bit MFMA routes take 16 / 32 / 64 / 128)")
    ap.add_argument("--grid", default=None, metavar="GHxGW",
                    help="rel-pos workloads: another token grid (T = GH * GW), e.g. 32x32")
    ap.add_argument("--batch", type=int, default=0, metavar="B",
                    help="override the workload's batch size (windowed workloads then draw plain random windows "
                         "instead of cutting them from one padded image); for scaling studies, not the headline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB per step (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU per process (asked for --gpus {args.gpus}); "
              "the path would shard by (batch, head) with no exchange, but no multi-GPU run exists.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_flash_sdpa_amd as fa
    import workloads

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    fa.load()
    if os.environ.get("SDPA_BENCH_UNFUSED", "0") == "1":
        fa.set_tuning("relpos_fused", 0)
    wl = workloads.WORKLOADS[args.workload]
    if args.dtype:
        if wl.dtype == "fp32":
            print("bench.py: --dtype applies to 16-bit workloads", file=sys.stderr)
            sys.exit(2)
        wl = wl.with_(dtype=args.dtype)
    if args.batch:
        if args.batch < 1:
            print("bench.py: --batch must be positive", file=sys.stderr)
            sys.exit(2)
        wl = wl.with_(B=args.batch, window_image=None)
    if args.head_dim:
        wl = wl.with_(D=args.head_dim)
    if args.grid:
        if not wl.relpos:
            print("bench.py: --grid needs a rel-pos workload", file=sys.stderr)
            sys.exit(2)
        gh, gw = (int(t) for t in args.grid.lower().split("x"))
        wl = wl.with_(grid=(gh, gw), Tq=gh * gw, Tkv=gh * gw, window_image=None)
    x = workloads.generate(wl, seed=0)
    g = {k: t.cuda() for k, t in x.items()}
    if args.pass_ == "backward":
        bench_backward(fa, wl, x, g, args)
        return
    if args.pass_ in ("dropout", "weights"):
        bench_train_forward(fa, wl, g, args)
        return
    if wl.relpos:
        n = fa.workspace_size(wl.B, wl.Hq, wl.Hkv, wl.Tq, wl.Tkv, wl.D, True, wl.grid, dtype=g["q"].dtype,
                              scale=wl.scale)
        if n:
            g["ws"] = torch.empty(n, dtype=torch.uint8, device="cuda")
    if args.route == "additive":
        if not wl.relpos:
            print("bench.py: --route additive needs a rel-pos workload", file=sys.stderr)
            sys.exit(2)
        th, tw = fa.relpos_terms(g["q"], g["rel_pos_h"], g["rel_pos_w"], wl.grid, layout=wl.layout)
        j = torch.arange(wl.grid[0] * wl.grid[1], device="cuda")
        g["bias"] = (th[..., j // wl.grid[1]] + tw[..., j % wl.grid[1]]).to(g["q"].dtype).contiguous()
        del th, tw, j
    torch.cuda.synchronize()

    # HBM-cold timing: working sets below the MALL's size cycle through >= 512 MiB of
    # buffer sets; the warm (one buffer set) times are reported beside them.
    sets = buffer_sets(g)
    warm = [sets[0]]
    sec = time_gpu(fa, wl, sets, args.steps, args.warmup)
    attn, bias = flop_model(wl)
    if args.route == "additive":
        bias = 2 * allowed_pairs(wl) * wl.B * wl.Hq      # the terms were formed before timing
    total = attn + bias
    tflops = total / sec / 1e12
    (call_ms, call_min), (terms_ms, terms_min) = kernel_events(fa, wl, sets, args.steps)
    (wcall_ms, wcall_min), (wterms_ms, _) = kernel_events(fa, wl, warm, args.steps)
    run_call(fa, wl, sets[0], sets[0]["out"])
    kernel = fa.last_kernel()
    rec_name = wl.name + ("_additive" if args.route == "additive" else "")
    if args.dtype and args.dtype != workloads.WORKLOADS[args.workload].dtype:
        rec_name += "_" + args.dtype
    if args.batch:
        rec_name += f"_b{args.batch}"
    if args.head_dim:
        rec_name += f"_d{args.head_dim}"
    if args.grid:
        rec_name += f"_g{args.grid.lower()}"
    traffic, traffic_src = recorded_traffic(kernel, rec_name)
    flash_ms = call_ms - terms_ms
    flash_flops = attn + (2 * allowed_pairs(wl) * wl.B * wl.Hq if wl.relpos else 0)
    if wl.relpos and terms_ms == 0.0:
        flash_flops = total             # terms formed inside the flash kernel: one launch per call
    achieved = flash_flops / (flash_ms * 1e-3) / 1e12
    set_bytes = sum(t.numel() * t.element_size() for t in sets[0].values())
    nbytes = byte_model(wl) + (g["bias"].numel() * g["bias"].element_size() if "bias" in g else 0)
    line = {
        "metric": "attention TFLOP/s + % bf16 MFMA peak, SAM ViT-B 64x64 global rel-pos SDPA",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp16": "f16"}.get(wl.dtype, "f32"),
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "layout": wl.layout, "B": wl.B,
                   "Hq": wl.Hq, "Hkv": wl.Hkv, "Tq": wl.Tq, "Tkv": wl.Tkv, "head_dim": wl.D,
                   "grid": list(wl.grid) if wl.grid else None, "mask": wl.mask, "scale": wl.scale,
                   "flop_per_step": total, "attn_flop": attn, "bias_flop": bias},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": kernel, "kernel_ms": round(flash_ms, 5),
                     "kernel_ms_min": round(call_min - terms_min, 5),
                     "terms_kernel_ms": round(terms_ms, 5), "flop_per_launch": flash_flops,
                     "algorithmic_bytes_per_launch": nbytes},
        "timing": {"cache": (f"HBM-cold: {len(sets)} buffer sets of {set_bytes} bytes cycled"
                             if len(sets) > 1 else "working set >= 256 MiB: one buffer set"),
                   "call_ms_median": round(call_ms, 5), "call_ms_min": round(call_min, 5),
                   "warm_call_ms_median": round(wcall_ms, 5), "warm_call_ms_min": round(wcall_min, 5),
                   "warm_tflops": round(total / (wcall_ms * 1e-3) / 1e12, 3),
                   "event_reps": 5, "calls_per_rep": args.steps},
    }
    if args.route == "additive":
        line["config"]["route"] = "additive mask (bias materialised before timing)"
    if args.route == "additive" or flash_flops / nbytes < MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        # Below the ridge (FLOPs per algorithmic byte under peak FLOP/s / peak bytes/s: decode
        # shapes, the windows, a materialised bias) HBM bounds the call: report it against HBM.
        gbs = nbytes / (flash_ms * 1e-3) / 1e9
        line["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(gbs / HBM_PEAK_GBS, 4), "attention_tflops": round(achieved, 3)})
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_budget)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
