"""Build the HIP shared library libsdpa.so in-tree for gfx950.

Every source under csrc/ is compiled with hipcc (one process per file, in
parallel) into _build/ and linked into attention_flash_sdpa_amd/libsdpa.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsdpa.so")
ARCH = os.environ.get("SDPA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of generated code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


# Per-file extra flags.  The MFMA attention kernels take row maxima of scores
# produced by the matrix cores; without NaN honouring the maxima need no
# quieting moves (NaN scores still reach the output through exp and P.V).
EXTRA = {f: ["-fno-honor-nans"] for f in ("flash_mfma.hip", "flash_split64.hip", "flash_split64w.hip", "flash_tiled.hip", "flash_window.hip")}
# Matrix-op accumulators in ordinary VGPRs: the tiled kernel's mask modes
# otherwise move them to AGPRs and lose a wave per SIMD.
EXTRA["flash_tiled.hip"] = EXTRA["flash_tiled.hip"] + ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip", f"--offload-arch={ARCH}"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + EXTRA.get(os.path.basename(src), []) + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj, out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, out in results:
        if verbose and out.strip():
            print(out, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
