"""CPU-side checks of the C ABI: the library loads, exports every function
include/sdpa.h declares, and rejects bad arguments before touching HIP."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import attention_flash_sdpa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", src, flags=re.M)) - {"defined"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sdpa_fwd", "sdpa_relpos_fwd", "relpos_terms", "sdpa_workspace_size",
              "sdpa_status_string", "sdpa_last_error", "sdpa_last_kernel", "sdpa_set_tuning",
              "sdpa_dropout_mask", "sdpa_fwd_dropout", "sdpa_bwd", "sdpa_bwd_workspace_size",
              "sdpa_attention_weights"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "sdpa.h"\nint main(void){ sdpa_mask m; (void)m; return (int)sizeof(sdpa_mask) - 64; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(tmp_path / "t")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(tmp_path / "t")]).returncode == 0      # struct is 64 bytes, as ctypes assumes
    assert ctypes.sizeof(fa._Mask) == 64


def call_fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dtype=1, out_dtype=1, layout=1, B=1, Hq=2, Hkv=2, Tq=8, Tkv=8,
             D=64, scale=float("nan"), mask=None, lse=None, ws=None, wsn=0, stream=None)
    a.update(kw)
    lib = fa.load()
    m = a["mask"]
    return lib.sdpa_fwd(a["q"], a["k"], a["v"], a["o"], a["dtype"], a["out_dtype"], a["layout"], a["B"], a["Hq"],
                        a["Hkv"], a["Tq"], a["Tkv"], a["D"], a["scale"], ctypes.byref(m) if m else None,
                        a["lse"], a["ws"], a["wsn"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(B=0), -1), (dict(Tq=-3), -1), (dict(D=0), -1),
    (dict(Hq=3, Hkv=2), -1), (dict(dtype=7), -1), (dict(out_dtype=7), -1), (dict(dtype=0, out_dtype=1), -1),
    (dict(layout=5), -1), (dict(D=48), -2), (dict(D=256), -2), (dict(dtype=0, out_dtype=0, D=200), -2),
])
def test_fwd_rejects(kw, status):
    assert call_fwd(**kw) == status
    assert fa.load().sdpa_last_error().decode() != ""


def test_fwd_rejects_bad_masks():
    m = fa._Mask()
    m.kind = 2
    m.window = 0
    assert call_fwd(mask=m) == -1 and b"window" in fa.load().sdpa_last_error()
    m = fa._Mask()
    m.kind = 3
    assert call_fwd(mask=m) == -1                 # additive without data
    m.data = 0x2000
    m.data_dtype = 9
    assert call_fwd(mask=m) == -1                 # bad additive dtype
    m = fa._Mask()
    m.kind = 4
    m.data = 0x2000
    m.stride[2] = -1
    assert call_fwd(mask=m) == -1
    m = fa._Mask()
    m.kind = 42
    assert call_fwd(mask=m) == -1


def test_relpos_rejects():
    lib = fa.load()
    args = [FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 8, 8, 64, FAKE, FAKE, float("nan"), None, None, 0, None]
    assert lib.sdpa_relpos_fwd(*args) == -3          # no workspace
    bad = list(args)
    bad[12] = None
    assert lib.sdpa_relpos_fwd(*bad) == -1           # missing table
    bad = list(args)
    bad[9] = 0
    assert lib.sdpa_relpos_fwd(*bad) == -1           # empty grid
    bad = list(args)
    bad[11] = 48
    assert lib.sdpa_relpos_fwd(*bad) == -2           # unsupported bf16 head_dim
    assert lib.relpos_terms(None, 1, 1, 1, 2, 8, 8, 64, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.relpos_terms(FAKE, 1, 1, 1, 2, 0, 8, 64, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.relpos_terms(FAKE, 3, 1, 1, 2, 8, 8, 64, FAKE, FAKE, FAKE, FAKE, None) == -1


def test_workspace_sizes():
    lib = fa.load()
    assert lib.sdpa_workspace_size(1, 12, 12, 4096, 4096, 64, 1, 64, 64) >= 1 * 12 * 4096 * 128 * 4
    assert lib.sdpa_workspace_size(1, 12, 12, 4096, 4096, 64, 1, 63, 64) == ctypes.c_size_t(-1).value
    assert lib.sdpa_workspace_size(0, 12, 12, 4096, 4096, 64, 0, 0, 0) == ctypes.c_size_t(-1).value
    assert lib.sdpa_workspace_size(4, 32, 8, 4096, 4096, 128, 0, 0, 0) == 0


def test_status_strings_and_tuning():
    lib = fa.load()
    assert lib.sdpa_status_string(0) == b"ok"
    assert lib.sdpa_status_string(-3) == b"workspace too small"
    assert lib.sdpa_set_tuning(b"nope", 1) == -1
    assert lib.sdpa_set_tuning(b"num_splits", -1) == -1
    assert lib.sdpa_set_tuning(b"num_splits", 0) == 0
    assert lib.sdpa_set_tuning(b"relpos_fused", 2) == -1
    assert lib.sdpa_set_tuning(b"split_wide", 3) == -1
    assert lib.sdpa_set_tuning(b"split_wide", 2) == 0
    assert lib.sdpa_set_tuning(b"split_wide", 1) == 0
    assert lib.sdpa_set_tuning(b"relpos_fused", 1) == 0
    assert lib.sdpa_relpos_fused(1, 64, 64, 64) == 1      # SAM ViT-B global grid: one kernel
    assert lib.sdpa_relpos_fused(1, 64, 14, 14) == 1      # SAM 14x14 window: one kernel
    assert lib.sdpa_relpos_fused(1, 64, 13, 14) == 1      # other small grids: generic kernel forms the terms
    assert lib.sdpa_relpos_fused(0, 16, 8, 8) == 1        # tiny fp32 grid: generic kernel forms the terms
    assert lib.sdpa_relpos_fused(1, 128, 64, 64) == 0     # tables too large to stage: terms kernel first
    assert lib.sdpa_relpos_fused(0, 64, 64, 64) == 0
    assert lib.sdpa_set_tuning(b"relpos_fused", 0) == 0
    assert lib.sdpa_relpos_fused(1, 64, 64, 64) == 0
    assert lib.sdpa_relpos_fused(1, 64, 14, 14) == 0
    assert lib.sdpa_set_tuning(b"relpos_fused", 1) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        fa.sdpa(x, x, x)


def test_default_scale():
    assert fa.default_scale(64) == 0.125 and math.isclose(fa.default_scale(128), 128 ** -0.5)


def test_last_kernel_starts_empty_per_thread():
    import threading
    lib = fa.load()
    got = []
    th = threading.Thread(target=lambda: got.append(lib.sdpa_last_kernel()))
    th.start()
    th.join()
    assert got == [b""]


def test_no_symbol_defined_in_two_objects():
    """Every externally visible function of the library comes from one object
    file: two sources defining the same (e.g. template) helper would silently
    resolve both call sites to one of them at link time."""
    build = os.path.join(ROOT, "attention_flash_sdpa_amd", "_build")
    objs = sorted(f for f in os.listdir(build) if f.endswith(".o")) if os.path.isdir(build) else []
    if not objs:
        pytest.skip("library objects not built here")
    seen = {}
    for f in objs:
        out = subprocess.run(["nm", "--defined-only", "-g", os.path.join(build, f)], capture_output=True, text=True).stdout
        for line in out.splitlines():
            parts = line.split()
            if len(parts) == 3 and parts[1] in "TWV" and "sdpa" in parts[2] and "__device_stub" not in parts[2]:
                assert parts[2] not in seen, f"{parts[2]} in {seen.get(parts[2])} and {f}"
                seen[parts[2]] = f


def test_training_entry_points_reject_bad_arguments():
    lib = fa.load()
    m = None
    # dropout mask: null output, bad rate, bad sizes
    assert lib.sdpa_dropout_mask(1, 0, 0.1, 1, 1, 8, 8, None, None) == -1
    assert lib.sdpa_dropout_mask(1, 0, 1.0, 1, 1, 8, 8, FAKE, None) == -1
    assert lib.sdpa_dropout_mask(1, 0, -0.1, 1, 1, 8, 8, FAKE, None) == -1
    assert lib.sdpa_dropout_mask(1, 0, float("nan"), 1, 1, 8, 8, FAKE, None) == -1
    assert lib.sdpa_dropout_mask(1, 0, 0.1, 1, 0, 8, 8, FAKE, None) == -1
    # dropout forward: keep bits are required, rate checked
    fwd = lambda keep, rate, **kw: lib.sdpa_fwd_dropout(FAKE, FAKE, FAKE, FAKE, kw.get("dtype", 1), kw.get("dtype", 1), 1,
                                                       1, 2, 2, 8, 8, kw.get("D", 64), float("nan"), m, keep, rate,
                                                       None, None, 0, None)
    assert fwd(None, 0.1) == -1
    assert fwd(FAKE, 1.5) == -1
    assert fwd(FAKE, 0.1, D=48) == -2
    # backward: required pointers, dtype support, workspace
    def bwd(**kw):
        a = dict(q=FAKE, lse=FAKE, dq=FAKE, dtype=1, odt=1, gdt=1, D=64, ws=FAKE, wsn=1 << 20, keep=None, rate=0.0)
        a.update(kw)
        return lib.sdpa_bwd(a["q"], FAKE, FAKE, FAKE, FAKE, a["lse"], a["dq"], FAKE, FAKE, a["dtype"], a["odt"],
                            a["gdt"], 1, 1, 2, 2, 8, 8, a["D"], float("nan"), m, a["keep"], a["rate"], a["ws"],
                            a["wsn"], None)
    assert bwd(q=None) == -1
    assert bwd(lse=None) == -1
    assert bwd(dq=None) == -1
    assert bwd(gdt=2) == -1                       # grads must be dtype or fp32
    assert bwd(dtype=0, odt=0, gdt=0) == -2       # fp32 inputs: not built
    assert bwd(D=16) == -2                        # head_dim 16: not built
    assert bwd(ws=None, wsn=0) == -3
    assert bwd(wsn=16) == -3
    assert bwd(keep=FAKE, rate=2.0) == -1
    assert lib.sdpa_bwd_workspace_size(2, 3, 100) == 2560
    assert lib.sdpa_bwd_workspace_size(0, 3, 100) == ctypes.c_size_t(-1).value
    # attention weights
    assert lib.sdpa_attention_weights(FAKE, FAKE, 1, 1, 1, 2, 2, 8, 8, 64, float("nan"), m, None, None, 0.0,
                                      FAKE, None) == -1
    assert lib.sdpa_attention_weights(FAKE, FAKE, 1, 1, 1, 2, 2, 8, 8, 64, float("nan"), m, FAKE, FAKE, 1.0,
                                      FAKE, None) == -1
