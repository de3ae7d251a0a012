"""MI355X-native fused scaled-dot-product attention (Python binding).

Thin ctypes layer over the C ABI in include/sdpa.h (libsdpa.so, built
in-tree for gfx950 by attention_flash_sdpa_amd/build.py).  This module only
marshals arguments: torch provides device memory and the current stream;
every step of the attention runs in the library's HIP kernels.  There is no
CPU fallback -- if the library or a GPU is missing, the calls raise.

    O = softmax(Q . K^T * scale + B) . V

[Axon PR 650] "Axon.Layers.scaled_dot_product_attention/4", description:
bshd (default) / bhsd layouts, scale defaulting to 1/sqrt(head_dim), causal /
sliding-window / tensor masks, grouped-query attention.
[mlx-examples issue 1451] "segment_anything: fuse attention with
mx.fast.scaled_dot_product_attention", body: SAM's decomposed rel-pos bias.
[Candle PR 3280] "feat(metal): SDPA with Relative Positional Embeddings &
LayerNorm Stability", Key Changes: term_h / term_w injected into the scores.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = ["load", "lib_path", "sdpa", "sdpa_noalloc", "sdpa_relpos", "relpos_terms", "workspace_size", "relpos_fused",
           "set_tuning", "dropout_mask", "sdpa_backward", "sdpa_relpos_backward", "attention_weights", "SdpaError", "F32", "BF16", "F16",
           "BSHD", "BHSD"]

F32, BF16, F16 = 0, 1, 2
BSHD, BHSD = 0, 1
_MASK_KIND = {"none": 0, "causal": 1, "sliding": 2, "additive": 3, "bool": 4}
_LAYOUT = {"bshd": BSHD, "bhsd": BHSD}
_DTYPE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_MASK_DTYPE = {torch.float32: F32, torch.bfloat16: BF16}


class SdpaError(RuntimeError):
    def __init__(self, status, where, detail):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class _Mask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("data_dtype", ctypes.c_int32),
                ("offset", ctypes.c_int64), ("window", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("stride", ctypes.c_int64 * 4)]


_LIB = None
_LOCK = threading.Lock()
_P, _I64, _I32, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float


def lib_path():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")


def load():
    """Load libsdpa.so (raises if it has not been built)."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with attention_flash_sdpa_amd/build.py")
        lib = ctypes.CDLL(path)
        lib.sdpa_workspace_size.restype = ctypes.c_size_t
        lib.sdpa_workspace_size.argtypes = [_I32] + [_I64] * 6 + [_F, _I32, _I64, _I64]
        lib.sdpa_fwd.restype = _I32
        lib.sdpa_fwd.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32] + [_I64] * 6 + \
            [_F, ctypes.POINTER(_Mask), _P, _P, ctypes.c_size_t, _P]
        lib.sdpa_fwd_noalloc.restype = _I32
        lib.sdpa_fwd_noalloc.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32] + [_I64] * 6 + \
            [_F, ctypes.POINTER(_Mask), _P, _P]
        lib.relpos_terms.restype = _I32
        lib.relpos_terms.argtypes = [_P, _I32, _I32] + [_I64] * 5 + [_P, _P, _P, _P, _P]
        lib.sdpa_relpos_fwd.restype = _I32
        lib.sdpa_relpos_fwd.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32] + [_I64] * 5 + \
            [_P, _P, _F, _P, _P, ctypes.c_size_t, _P]
        lib.sdpa_status_string.restype = ctypes.c_char_p
        lib.sdpa_status_string.argtypes = [_I32]
        lib.sdpa_last_error.restype = ctypes.c_char_p
        lib.sdpa_last_error.argtypes = []
        lib.sdpa_last_kernel.restype = ctypes.c_char_p
        lib.sdpa_last_kernel.argtypes = []
        lib.sdpa_set_tuning.restype = _I32
        lib.sdpa_set_tuning.argtypes = [ctypes.c_char_p, _I64]
        lib.sdpa_relpos_fused.restype = _I32
        lib.sdpa_relpos_fused.argtypes = [_I32, _I64, _I64, _I64]
        lib.sdpa_dropout_mask.restype = _I32
        lib.sdpa_dropout_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint32, _F] + [_I64] * 4 + [_P, _P]
        lib.sdpa_fwd_dropout.restype = _I32
        lib.sdpa_fwd_dropout.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32] + [_I64] * 6 + \
            [_F, ctypes.POINTER(_Mask), _P, _F, _P, _P, ctypes.c_size_t, _P]
        lib.sdpa_bwd_workspace_size.restype = ctypes.c_size_t
        lib.sdpa_bwd_workspace_size.argtypes = [_I64] * 3
        lib.sdpa_bwd.restype = _I32
        lib.sdpa_bwd.argtypes = [_P] * 9 + [_I32] * 4 + [_I64] * 6 + \
            [_F, ctypes.POINTER(_Mask), _P, _F, _P, ctypes.c_size_t, _P]
        lib.sdpa_relpos_bwd_workspace_size.restype = ctypes.c_size_t
        lib.sdpa_relpos_bwd_workspace_size.argtypes = [_I64] * 5
        lib.sdpa_relpos_bwd.restype = _I32
        lib.sdpa_relpos_bwd.argtypes = [_P] * 11 + [_I32] * 4 + [_I64] * 5 + [_P, _P, _F, _P, ctypes.c_size_t, _P]
        lib.sdpa_relpos_bwd_dropout.restype = _I32
        lib.sdpa_relpos_bwd_dropout.argtypes = [_P] * 11 + [_I32] * 4 + [_I64] * 5 + \
            [_P, _P, _F, _P, _F, _P, ctypes.c_size_t, _P]
        lib.sdpa_relpos_fwd_dropout_workspace_size.restype = ctypes.c_size_t
        lib.sdpa_relpos_fwd_dropout_workspace_size.argtypes = [_I64] * 4
        lib.sdpa_relpos_fwd_dropout.restype = _I32
        lib.sdpa_relpos_fwd_dropout.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32] + [_I64] * 5 + \
            [_P, _P, _F, _P, _F, _P, _P, ctypes.c_size_t, _P]
        lib.sdpa_attention_weights.restype = _I32
        lib.sdpa_attention_weights.argtypes = [_P, _P, _I32, _I32] + [_I64] * 6 + \
            [_F, ctypes.POINTER(_Mask), _P, _P, _F, _P, _P]
        _LIB = lib
        return lib


def _check(status, where):
    if status != 0:
        lib = load()
        detail = lib.sdpa_last_error().decode() or lib.sdpa_status_string(status).decode()
        raise SdpaError(status, where, detail)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU path exists)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous in the stated layout")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def last_kernel():
    """Name of the attention kernel the last successful call on this thread launched."""
    return load().sdpa_last_kernel().decode()


def set_tuning(key, value):
    """Process-wide knob: "num_splits" (0 = auto), "split_halves", "tiled" or "relpos_fused" (0/1)."""
    _check(load().sdpa_set_tuning(key.encode(), int(value)), "sdpa_set_tuning")


def relpos_fused(dtype, D, grid):
    """True if sdpa_relpos runs as a single kernel that forms the terms itself."""
    return bool(load().sdpa_relpos_fused(_DTYPE[dtype], D, grid[0], grid[1]))


def workspace_size(B, Hq, Hkv, Tq, Tkv, D, relpos=False, grid=(0, 0), dtype=torch.bfloat16, scale=None):
    """Device workspace bytes of sdpa (relpos=False) or sdpa_relpos for these sizes and dtype."""
    sc = float("nan") if scale is None else float(scale)
    n = load().sdpa_workspace_size(_DTYPE[dtype], B, Hq, Hkv, Tq, Tkv, D, sc, int(bool(relpos)), grid[0], grid[1])
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for sdpa_workspace_size")
    return n


def _layout_of(layout):
    if layout not in _LAYOUT:
        raise ValueError(f"layout must be 'bhsd' or 'bshd' (got {layout!r})")
    return _LAYOUT[layout]


def _dims(q, k, layout):
    """(B, Hq, Hkv, Tq, Tkv, D) of rank-4 q and k in the layout; q and k must agree on B and D."""
    _layout_of(layout)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be rank-4")
    if layout == "bhsd":
        B, Hq, Tq, D = q.shape
        Bk, Hkv, Tkv, Dk = k.shape
    else:
        B, Tq, Hq, D = q.shape
        Bk, Tkv, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree on batch or head_dim ({layout})")
    return B, Hq, Hkv, Tq, Tkv, D


def _expect(name, t, shape, dtype, device):
    """t must be a contiguous tensor of exactly this shape and dtype on q's device."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_qkv(q, k, v, layout):
    """Shapes, dtypes and devices of q, k, v (before any launch); returns the sizes."""
    if q.dtype not in _DTYPE:
        raise ValueError("q, k, v must be float32, bfloat16 or float16")
    dims = _dims(q, k, layout)
    _expect("k", k, tuple(k.shape), q.dtype, q.device)
    _expect("v", v, tuple(k.shape), q.dtype, q.device)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    return dims


def _check_tables(rel_pos_h, rel_pos_w, grid, D, q):
    gh, gw = grid
    _expect("rel_pos_h", rel_pos_h, (2 * gh - 1, D), q.dtype, q.device)
    _expect("rel_pos_w", rel_pos_w, (2 * gw - 1, D), q.dtype, q.device)


def _relpos_dims(q, k, v, grid, layout):
    B, H, Hkv, T, Tkv, D = _check_qkv(q, k, v, layout)
    gh, gw = grid
    if Hkv != H or Tkv != T:
        raise ValueError("rel-pos attention is self-attention: k and v must be shaped like q")
    if gh <= 0 or gw <= 0 or gh * gw != T:
        raise ValueError(f"grid {grid} does not match the sequence length {T}")
    return B, H, T, D


def _mask_struct(mask, B, Hq, Tq, Tkv, keep, device):
    m = _Mask()
    m.kind = 0
    if mask is None:
        return m
    kind = mask["kind"]
    if kind not in _MASK_KIND:
        raise ValueError(f"unknown mask kind {kind!r}")
    m.kind = _MASK_KIND[kind]
    m.offset = int(mask.get("offset", 0))
    m.window = int(mask.get("window", 0))
    if kind in ("additive", "bool"):
        data = mask["data"]
        if data.dim() != 4:
            raise ValueError("tensor masks are rank-4, broadcastable to [B, Hq, Tq, Tkv]")
        try:
            torch.broadcast_shapes(tuple(data.shape), (B, Hq, Tq, Tkv))
        except RuntimeError:
            raise ValueError(f"mask of shape {tuple(data.shape)} does not broadcast to {(B, Hq, Tq, Tkv)}") from None
        if data.device != device:
            raise ValueError(f"mask is on {data.device}, expected {device} (no CPU path exists)")
        if kind == "bool":
            if data.dtype != torch.bool:
                raise ValueError("bool masks must be torch.bool")
            data = data.view(torch.uint8)
        else:
            if data.dtype not in _MASK_DTYPE:
                raise ValueError("additive masks must be float32 or bfloat16")
            m.data_dtype = _MASK_DTYPE[data.dtype]
        ex = data.expand(B, Hq, Tq, Tkv)
        for a in range(4):
            m.stride[a] = ex.stride(a)
        m.data = data.data_ptr()
        keep.append(data)
    return m


def _dropout_args(dropout, B, Hq, Tq, Tkv):
    """(keep pointer, rate) from {"keep": int32 words [B, Hq, Tq, ceil(Tkv/32)], "rate": r} or None."""
    if dropout is None:
        return None, 0.0
    keep = dropout["keep"]
    if tuple(keep.shape) != (B, Hq, Tq, (Tkv + 31) // 32):
        raise ValueError(f"dropout keep bits have shape {tuple(keep.shape)}, expected {(B, Hq, Tq, (Tkv + 31) // 32)}")
    if not keep.is_cuda or keep.dtype != torch.int32 or not keep.is_contiguous():
        raise ValueError("dropout keep bits must be a contiguous int32 GPU tensor (from dropout_mask)")
    return _ptr(keep), float(dropout["rate"])


def _check_bwd_io(q, o, dout, lse, B, Hq, Tq):
    if o.dtype not in (q.dtype, torch.float32):
        raise ValueError("o must be in q's dtype or float32")
    _expect("o", o, tuple(q.shape), o.dtype, q.device)
    _expect("dout", dout, tuple(q.shape), q.dtype, q.device)
    _expect("lse", lse, (B, Hq, Tq), torch.float32, q.device)


def sdpa(q, k, v, *, layout="bhsd", scale=None, mask=None, out_dtype=None, return_lse=False,
         stream=None, out=None, dropout=None):
    """Fused attention on the GPU.

    q: [B, Hq, Tq, D] (bhsd) or [B, Tq, Hq, D] (bshd); k, v with Hkv heads.
    mask: None | {"kind": "causal", "offset": d} | {"kind": "sliding", "window": w, "offset": d}
          | {"kind": "additive", "data": tensor} | {"kind": "bool", "data": bool tensor}
    out_dtype: None (= q.dtype) or torch.float32.
    dropout: None | {"keep": keep bits from dropout_mask, "rate": r} (attention dropout).
    """
    lib = load()
    B, Hq, Hkv, Tq, Tkv, D = _check_qkv(q, k, v, layout)
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in (q.dtype, torch.float32):
        raise ValueError("out_dtype must be q's dtype or torch.float32")
    if out is not None:
        _expect("out", out, tuple(q.shape), odt, q.device)
    _need_gpu(q, k, v)
    o = out if out is not None else torch.empty(q.shape, dtype=odt, device=q.device)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if return_lse else None
    keep = []
    ms = _mask_struct(mask, B, Hq, Tq, Tkv, keep, q.device)
    sc = float("nan") if scale is None else float(scale)
    ws_n = lib.sdpa_workspace_size(_DTYPE[q.dtype], B, Hq, Hkv, Tq, Tkv, D, sc, 0, 0, 0)
    if ws_n == ctypes.c_size_t(-1).value:
        ws_n = 0                      # sizes the library refuses: the call below reports why
    ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device) if ws_n else None
    if dropout is not None:
        kp, rate = _dropout_args(dropout, B, Hq, Tq, Tkv)
        st = lib.sdpa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _DTYPE[q.dtype], _DTYPE[odt],
                                  _layout_of(layout), B, Hq, Hkv, Tq, Tkv, D, sc, ctypes.byref(ms), kp, rate,
                                  _ptr(lse), None, 0, _stream(stream))
        _check(st, "sdpa_fwd_dropout")
        return (o, lse) if return_lse else o
    st = lib.sdpa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _DTYPE[q.dtype], _DTYPE[odt], _layout_of(layout),
                      B, Hq, Hkv, Tq, Tkv, D, sc, ctypes.byref(ms), _ptr(lse), _ptr(ws), ws_n, _stream(stream))
    _check(st, "sdpa_fwd")
    return (o, lse) if return_lse else o


def sdpa_noalloc(q, k, v, out, *, layout="bhsd", scale=None, mask=None, lse=None, stream=None):
    """sdpa into the caller's `out` (and optional `lse` [B, Hq, Tq] fp32) through the
    allocation-free entry point: neither the library nor this wrapper allocates."""
    lib = load()
    B, Hq, Hkv, Tq, Tkv, D = _check_qkv(q, k, v, layout)
    if out.dtype not in (q.dtype, torch.float32):
        raise ValueError("out must be in q's dtype or torch.float32")
    _expect("out", out, tuple(q.shape), out.dtype, q.device)
    if lse is not None:
        _expect("lse", lse, (B, Hq, Tq), torch.float32, q.device)
    _need_gpu(q, k, v)
    ms = _mask_struct(mask, B, Hq, Tq, Tkv, [], q.device)
    sc = float("nan") if scale is None else float(scale)
    st = lib.sdpa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _DTYPE[q.dtype], _DTYPE[out.dtype],
                              _layout_of(layout), B, Hq, Hkv, Tq, Tkv, D, sc, ctypes.byref(ms), _ptr(lse),
                              _stream(stream))
    _check(st, "sdpa_fwd_noalloc")
    return out


def dropout_mask(seed, step, rate, B, Hq, Tq, Tkv, *, device="cuda", stream=None):
    """Dropout keep bits [B, Hq, Tq, ceil(Tkv / 32)] as int32 words (Philox4x32-10 of (seed, step))."""
    lib = load()
    keep = torch.empty((B, Hq, Tq, (Tkv + 31) // 32), dtype=torch.int32, device=device)
    st = lib.sdpa_dropout_mask(int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, float(rate), B, Hq, Tq, Tkv,
                               _ptr(keep), _stream(stream))
    _check(st, "sdpa_dropout_mask")
    return keep


def sdpa_backward(q, k, v, o, dout, lse, *, layout="bhsd", scale=None, mask=None, dropout=None,
                  grad_dtype=None, stream=None):
    """(dq, dk, dv) of attention for the upstream gradient dout (o and lse from the forward call)."""
    lib = load()
    B, Hq, Hkv, Tq, Tkv, D = _check_qkv(q, k, v, layout)
    _check_bwd_io(q, o, dout, lse, B, Hq, Tq)
    _need_gpu(q, k, v, o, dout, lse)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    if gdt not in (q.dtype, torch.float32):
        raise ValueError("grad_dtype must be q's dtype or torch.float32")
    dq = torch.empty(q.shape, dtype=gdt, device=q.device)
    dk = torch.empty(k.shape, dtype=gdt, device=q.device)
    dv = torch.empty(v.shape, dtype=gdt, device=q.device)
    keep_refs = []
    ms = _mask_struct(mask, B, Hq, Tq, Tkv, keep_refs, q.device)
    kp, rate = _dropout_args(dropout, B, Hq, Tq, Tkv)
    ws_n = lib.sdpa_bwd_workspace_size(B, Hq, Tq)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    sc = float("nan") if scale is None else float(scale)
    st = lib.sdpa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      _DTYPE[q.dtype], _DTYPE[o.dtype], _DTYPE[gdt], _layout_of(layout), B, Hq, Hkv, Tq, Tkv, D, sc,
                      ctypes.byref(ms), kp, rate, _ptr(ws), ws_n, _stream(stream))
    _check(st, "sdpa_bwd")
    return dq, dk, dv


def sdpa_relpos_backward(q, k, v, o, dout, lse, rel_pos_h, rel_pos_w, grid, *, layout="bhsd", scale=None,
                         grad_dtype=None, stream=None, workspace=None, dropout=None):
    """(dq, dk, dv, d_rel_pos_h, d_rel_pos_w) of sdpa_relpos (tables' gradients in float32).
    dropout: None or the {"keep", "rate"} given to the forward call."""
    lib = load()
    B, H, T, D = _relpos_dims(q, k, v, grid, layout)
    gh, gw = grid
    _check_tables(rel_pos_h, rel_pos_w, grid, D, q)
    _check_bwd_io(q, o, dout, lse, B, H, T)
    _need_gpu(q, k, v, o, dout, lse, rel_pos_h, rel_pos_w)
    gdt = q.dtype if grad_dtype is None else grad_dtype
    if gdt not in (q.dtype, torch.float32):
        raise ValueError("grad_dtype must be q's dtype or torch.float32")
    dq = torch.empty(q.shape, dtype=gdt, device=q.device)
    dk = torch.empty(k.shape, dtype=gdt, device=q.device)
    dv = torch.empty(v.shape, dtype=gdt, device=q.device)
    drh = torch.empty(tuple(rel_pos_h.shape), dtype=torch.float32, device=q.device)
    drw = torch.empty(tuple(rel_pos_w.shape), dtype=torch.float32, device=q.device)
    ws_n = lib.sdpa_relpos_bwd_workspace_size(B, H, gh, gw, D)
    if ws_n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for sdpa_relpos_bwd")
    ws = workspace
    if ws is None or ws.numel() < ws_n:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    elif ws.dtype != torch.uint8 or ws.device != q.device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    sc = float("nan") if scale is None else float(scale)
    if dropout is not None:
        kp, rate = _dropout_args(dropout, B, H, T, T)
        st = lib.sdpa_relpos_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                         _ptr(dk), _ptr(dv), _ptr(drh), _ptr(drw), _DTYPE[q.dtype], _DTYPE[o.dtype],
                                         _DTYPE[gdt], _layout_of(layout), B, H, gh, gw, D, _ptr(rel_pos_h),
                                         _ptr(rel_pos_w), sc, kp, rate, _ptr(ws), ws.numel(), _stream(stream))
        _check(st, "sdpa_relpos_bwd_dropout")
        return dq, dk, dv, drh, drw
    st = lib.sdpa_relpos_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(drh), _ptr(drw), _DTYPE[q.dtype], _DTYPE[o.dtype], _DTYPE[gdt], _layout_of(layout),
                             B, H, gh, gw, D, _ptr(rel_pos_h), _ptr(rel_pos_w), sc, _ptr(ws), ws.numel(),
                             _stream(stream))
    _check(st, "sdpa_relpos_bwd")
    return dq, dk, dv, drh, drw


def attention_weights(q, k, lse, *, layout="bhsd", scale=None, mask=None, dropout=None, stream=None):
    """[B, Hq, Tq, Tkv] fp32 weights that multiply V (lse from the forward call on the same inputs)."""
    lib = load()
    if q.dtype not in _DTYPE:
        raise ValueError("q, k must be float32, bfloat16 or float16")
    B, Hq, Hkv, Tq, Tkv, D = _dims(q, k, layout)
    _expect("k", k, tuple(k.shape), q.dtype, q.device)
    _expect("lse", lse, (B, Hq, Tq), torch.float32, q.device)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _need_gpu(q, k, lse)
    w = torch.empty((B, Hq, Tq, Tkv), dtype=torch.float32, device=q.device)
    keep_refs = []
    ms = _mask_struct(mask, B, Hq, Tq, Tkv, keep_refs, q.device)
    kp, rate = _dropout_args(dropout, B, Hq, Tq, Tkv)
    sc = float("nan") if scale is None else float(scale)
    st = lib.sdpa_attention_weights(_ptr(q), _ptr(k), _DTYPE[q.dtype], _layout_of(layout), B, Hq, Hkv, Tq, Tkv, D,
                                    sc, ctypes.byref(ms), _ptr(lse), kp, rate, _ptr(w), _stream(stream))
    _check(st, "sdpa_attention_weights")
    return w


def relpos_terms(q, rel_pos_h, rel_pos_w, grid, *, layout="bhsd", stream=None):
    """term_h [B, H, T, grid_h], term_w [B, H, T, grid_w] (fp32) on the GPU."""
    lib = load()
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float32, bfloat16 or float16")
    _layout_of(layout)
    if q.dim() != 4:
        raise ValueError("q must be rank-4")
    gh, gw = grid
    if layout == "bhsd":
        B, H, T, D = q.shape
    else:
        B, T, H, D = q.shape
    if gh <= 0 or gw <= 0 or gh * gw != T:
        raise ValueError(f"grid {grid} does not match the sequence length {T}")
    _check_tables(rel_pos_h, rel_pos_w, grid, D, q)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _need_gpu(q, rel_pos_h, rel_pos_w)
    th = torch.empty((B, H, T, gh), dtype=torch.float32, device=q.device)
    tw = torch.empty((B, H, T, gw), dtype=torch.float32, device=q.device)
    st = lib.relpos_terms(_ptr(q), _DTYPE[q.dtype], _layout_of(layout), B, H, gh, gw, D,
                          _ptr(rel_pos_h), _ptr(rel_pos_w), _ptr(th), _ptr(tw), _stream(stream))
    _check(st, "relpos_terms")
    return th, tw


def sdpa_relpos(q, k, v, rel_pos_h, rel_pos_w, grid, *, layout="bhsd", scale=None, out_dtype=None,
                return_lse=False, stream=None, out=None, workspace=None, dropout=None):
    """Fused attention with the decomposed rel-pos bias (self-attention on a grid).
    dropout: None | {"keep": keep bits from dropout_mask(.., B, H, T, T), "rate": r}."""
    lib = load()
    B, H, T, D = _relpos_dims(q, k, v, grid, layout)
    gh, gw = grid
    _check_tables(rel_pos_h, rel_pos_w, grid, D, q)
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in (q.dtype, torch.float32):
        raise ValueError("out_dtype must be q's dtype or torch.float32")
    if out is not None:
        _expect("out", out, tuple(q.shape), odt, q.device)
    _need_gpu(q, k, v, rel_pos_h, rel_pos_w)
    o = out if out is not None else torch.empty(q.shape, dtype=odt, device=q.device)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    sc = float("nan") if scale is None else float(scale)
    if dropout is not None:
        ws_n = lib.sdpa_relpos_fwd_dropout_workspace_size(B, H, gh, gw)
    else:
        ws_n = lib.sdpa_workspace_size(_DTYPE[q.dtype], B, H, H, T, T, D, sc, 1, gh, gw)
    if ws_n == ctypes.c_size_t(-1).value:
        raise ValueError("grid does not match the sequence length")
    ws = workspace
    if ws_n == 0:
        ws = None                     # the fused route needs no workspace
    elif ws is None or ws.numel() < ws_n:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    elif ws.dtype != torch.uint8 or ws.device != q.device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    if dropout is not None:
        kp, rate = _dropout_args(dropout, B, H, T, T)
        st = lib.sdpa_relpos_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _DTYPE[q.dtype], _DTYPE[odt],
                                         _layout_of(layout), B, H, gh, gw, D, _ptr(rel_pos_h), _ptr(rel_pos_w), sc,
                                         kp, rate, _ptr(lse), _ptr(ws), ws.numel(), _stream(stream))
        _check(st, "sdpa_relpos_fwd_dropout")
        return (o, lse) if return_lse else o
    st = lib.sdpa_relpos_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _DTYPE[q.dtype], _DTYPE[odt],
                             _layout_of(layout), B, H, gh, gw, D, _ptr(rel_pos_h), _ptr(rel_pos_w), sc,
                             _ptr(lse), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream))
    _check(st, "sdpa_relpos_fwd")
    return (o, lse) if return_lse else o


def default_scale(D):
    """[Axon PR 650], description: the scale defaults to 1/sqrt(head_dim)."""
    return 1.0 / math.sqrt(D)
