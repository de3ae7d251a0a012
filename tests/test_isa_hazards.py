"""Every kernel's gfx950 assembly keeps enough wait states between each matrix
op and any instruction that reads or overwrites its result, along every
control-flow path (see isa_hazards.py).  Compiles each HIP source to assembly
with the library's own flags; needs hipcc, no GPU."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

import isa_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_flash_sdpa_amd", "csrc")


def _asm(src, out_dir):
    from attention_flash_sdpa_amd import build as b
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [b.hipcc()] + b.COMMON + b.EXTRA.get(os.path.basename(src), []) + \
        ["-x", "hip", f"--offload-arch={b.ARCH}", "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=8) as ex:
        return dict(zip((os.path.basename(s) for s in srcs), ex.map(lambda s: _asm(s, d), srcs)))


def test_checker_finds_a_planted_hazard():
    """A read three instructions behind the op, reached around a divergent branch."""
    asm = """_Zk:
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], 0
\ts_and_saveexec_b64 s[0:1], vcc
\ts_cbranch_execz .LBB0_2
\tv_mov_b32_e32 v8, v9
\ts_nop 7
\ts_nop 7
.LBB0_2:
\ts_or_b64 exec, exec, s[0:1]
\tv_accvgpr_read_b32 v17, a15
\ts_endpgm
"""
    found = isa_hazards.hazards(isa_hazards.functions(asm)["_Zk"])
    assert len(found) == 1 and found[0][2] == 3
    assert not isa_hazards.hazards(isa_hazards.functions(asm.replace("\ts_or_b64", "\ts_nop 7\n\ts_or_b64"))["_Zk"])


def test_no_matrix_op_hazards(assembly):
    bad = []
    for name, path in assembly.items():
        with open(path) as f:
            for fn, items in isa_hazards.functions(f.read()).items():
                for h in isa_hazards.hazards(items):
                    bad.append(f"{name} {fn[:60]}: {h[0]} -> {h[1]} after {h[2]} wait states")
    assert not bad, "\n".join(bad[:20])
