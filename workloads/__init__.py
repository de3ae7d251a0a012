"""Seeded synthetic inputs for the attention workloads (no attention arithmetic).

Both the HIP library's tests/benchmark and the CPU oracle consume these
tensors; this module only draws random numbers, rounds them to the storage
dtype and lays them out.  It computes nothing of the attention method.

Workloads (shapes after the pages' models: SAM's image encoder and mask
decoder, and the masked / grouped-query options of the Axon kernel):

  tiny_relpos_fp32      fp32 bhsd B1 H2 T64 (8x8 grid) D16, rel-pos tables [15,16], scale 1/4
  sam_decoder_q7        bf16 bhsd B1 H8 D16, T_q 7 x T_kv 4096, no mask, scale 1/4
  sam_decoder_kv7       bf16 bhsd B1 H8 D16, T_q 4096 x T_kv 7, no mask, scale 1/4
  sam_window_relpos     bf16 bhsd 25 windows x H12 x T196 (14x14) D64, tables [27,64], scale 1/8
  sam_global_relpos     bf16 bhsd B1 H12 T4096 (64x64 grid) D64, tables [127,64], scale 1/8
  gqa_causal            bf16 bshd B4 Hq32 Hkv8 S4096 D128, causal, scale 1/sqrt(128)
  gqa_sliding           same inputs, causal + sliding window 1024
  gqa_decode            the same model's decode step: bshd B4 Hq32 Hkv8, one new query per
                        sequence against a 4096-token K/V cache (causal, offset 4095), D128

Generator: numpy PCG64 `default_rng(seed)`, `standard_normal(shape, float32)`
drawn in the order Q, K, V, rel_pos_h, rel_pos_w in the logical [B, H, T, D]
order; the tables are scaled by 0.02 (standard deviation); values are then
rounded to the storage dtype (round-to-nearest-even through torch) and
permuted to the workload's layout.  The windowed SAM workload draws its
tokens on the 64x64 image grid ([1, 64, 64, H, D]), zero-pads the grid to
70x70 and cuts it into 5x5 windows of 14x14 tokens, windows in row-major
order and tokens row-major inside a window.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "generate", "replica"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "fp32" | "bf16"
    layout: str           # "bhsd" | "bshd"
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tkv: int
    D: int
    scale: float
    mask: dict | None = None          # {"kind": "causal"|"sliding", "window": w, "offset": d}
    grid: tuple | None = None         # (grid_h, grid_w) for rel-pos
    window_image: tuple | None = None  # (image_side, padded_side, window_side) for windowed SAM
    description: str = ""

    @property
    def relpos(self):
        return self.grid is not None

    def with_(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_relpos_fp32": Workload(
        "tiny_relpos_fp32", "fp32", "bhsd", 1, 2, 2, 64, 64, 16, 0.25, grid=(8, 8),
        description="tiny rel-pos SDPA, fp32, 8x8 grid"),
    "sam_decoder_q7": Workload(
        "sam_decoder_q7", "bf16", "bhsd", 1, 8, 8, 7, 4096, 16, 0.25,
        description="SAM mask-decoder cross attention, 7 tokens attending 4096 image tokens"),
    "sam_decoder_kv7": Workload(
        "sam_decoder_kv7", "bf16", "bhsd", 1, 8, 8, 4096, 7, 16, 0.25,
        description="SAM mask-decoder cross attention, 4096 image tokens attending 7 tokens"),
    "sam_window_relpos": Workload(
        "sam_window_relpos", "bf16", "bhsd", 25, 12, 12, 196, 196, 64, 0.125, grid=(14, 14),
        window_image=(64, 70, 14),
        description="SAM ViT-B windowed rel-pos attention, 25 windows of 14x14"),
    "sam_global_relpos": Workload(
        "sam_global_relpos", "bf16", "bhsd", 1, 12, 12, 4096, 4096, 64, 0.125, grid=(64, 64),
        description="SAM ViT-B global rel-pos attention, 64x64 grid"),
    "gqa_causal": Workload(
        "gqa_causal", "bf16", "bshd", 4, 32, 8, 4096, 4096, 128, 1.0 / math.sqrt(128),
        mask={"kind": "causal", "offset": 0},
        description="decoder-style GQA 4:1, causal"),
    "gqa_sliding": Workload(
        "gqa_sliding", "bf16", "bshd", 4, 32, 8, 4096, 4096, 128, 1.0 / math.sqrt(128),
        mask={"kind": "sliding", "window": 1024, "offset": 0},
        description="decoder-style GQA 4:1, causal + sliding window 1024"),
    "gqa_decode": Workload(
        "gqa_decode", "bf16", "bshd", 4, 32, 8, 1, 4096, 128, 1.0 / math.sqrt(128),
        mask={"kind": "causal", "offset": 4095},
        description="decode step of the decoder-style GQA 4:1 model: one query against a 4096-token cache"),
}

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def _round(x, dtype):
    """float32 numpy -> torch tensor in the storage dtype (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPE[dtype])


def _layout(x_bhsd, layout):
    if layout == "bhsd":
        return x_bhsd.contiguous()
    return x_bhsd.permute(0, 2, 1, 3).contiguous()


def _windowed(rng, wl, H, D):
    img, pad, win = wl.window_image
    tok = rng.standard_normal((1, img, img, H, D), dtype=np.float32)
    full = np.zeros((1, pad, pad, H, D), dtype=np.float32)
    full[:, :img, :img] = tok
    nw = pad // win
    x = full.reshape(1, nw, win, nw, win, H, D).transpose(0, 1, 3, 2, 4, 5, 6)
    x = x.reshape(nw * nw, win * win, H, D)          # [windows, T, H, D]
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3))  # logical [B, H, T, D]


def generate(wl, seed=0, layout=None):
    """Draw the inputs of workload `wl` (a Workload or its name).

    Returns a dict of CPU torch tensors in the storage dtype and layout:
    q, k, v and, for rel-pos workloads, rel_pos_h and rel_pos_w ([2g-1, D]).
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    layout = layout or wl.layout
    rng = np.random.default_rng(seed)
    if wl.window_image is not None:
        q = _windowed(rng, wl, wl.Hq, wl.D)
        k = _windowed(rng, wl, wl.Hkv, wl.D)
        v = _windowed(rng, wl, wl.Hkv, wl.D)
        if q.shape[0] != wl.B or q.shape[2] != wl.Tq:
            raise ValueError("window recipe does not match the workload shape")
    else:
        q = rng.standard_normal((wl.B, wl.Hq, wl.Tq, wl.D), dtype=np.float32)
        k = rng.standard_normal((wl.B, wl.Hkv, wl.Tkv, wl.D), dtype=np.float32)
        v = rng.standard_normal((wl.B, wl.Hkv, wl.Tkv, wl.D), dtype=np.float32)
    out = {"q": _layout(_round(q, wl.dtype), layout),
           "k": _layout(_round(k, wl.dtype), layout),
           "v": _layout(_round(v, wl.dtype), layout)}
    if wl.relpos:
        gh, gw = wl.grid
        rh = 0.02 * rng.standard_normal((2 * gh - 1, wl.D), dtype=np.float32)
        rw = 0.02 * rng.standard_normal((2 * gw - 1, wl.D), dtype=np.float32)
        out["rel_pos_h"] = _round(rh, wl.dtype)
        out["rel_pos_w"] = _round(rw, wl.dtype)
    return out


def replica(name, **overrides):
    """A small copy of a workload that the oracle finishes in seconds but that
    still spans several kernel tiles and a ragged tail."""
    wl = WORKLOADS[name]
    small = {
        "tiny_relpos_fp32": {},
        "sam_decoder_q7": dict(Tkv=1000),
        "sam_decoder_kv7": dict(Tq=1000),
        "sam_window_relpos": dict(B=2, Hq=3, Hkv=3, window_image=None),
        "sam_global_relpos": dict(Hq=2, Hkv=2, Tq=16 * 64, Tkv=16 * 64, grid=(16, 64)),
        "gqa_causal": dict(B=1, Hq=8, Hkv=2, Tq=333, Tkv=333),
        "gqa_sliding": dict(B=1, Hq=8, Hkv=2, Tq=333, Tkv=333,
                            mask={"kind": "sliding", "window": 100, "offset": 0}),
        "gqa_decode": dict(B=2, Hq=8, Hkv=2, Tq=3, Tkv=1000, mask={"kind": "causal", "offset": 997}),
    }[name]
    small.update(overrides)
    return wl.with_(**small)
