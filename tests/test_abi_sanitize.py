"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp is compiled for the host only, with both sanitizers, and linked with
the library's kernel objects into tests/abi_sanitize_driver.c, a C program
that calls every entry point with arguments that validation must turn away
(null pointers, bad enums, non-positive and extreme sizes, oversized
grids, masks and dropout rates) and sweeps the workspace-size queries over
extreme values.  No call reaches a HIP launch, so this runs without a GPU;
any out-of-bounds access, signed overflow or bad shift in the host code
aborts the program with the sanitizer's report.
"""
import os
import shutil
import subprocess

import pytest

import attention_flash_sdpa_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_flash_sdpa_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1"]


def _kernel_objects():
    build = os.path.join(PKG, "_build")
    if not os.path.isdir(build):
        return []
    return sorted(os.path.join(build, f) for f in os.listdir(build)
                  if f.endswith(".o") and f != "abi.cpp.o")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("no host C/C++ compiler")
    fa.load()                                       # the kernel objects exist once the library is built
    objs = _kernel_objects()
    if not objs:
        pytest.skip("library objects not built")
    d = tmp_path_factory.mktemp("abi_san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-I", os.path.join(ROCM, "include")]
    _run(["gcc", "-std=c99", "-Wall", "-Werror"] + SAN + inc +
         ["-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), "-o", "drv.o"], d)
    _run(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__"] + SAN + inc +
         ["-c", os.path.join(PKG, "csrc", "abi.cpp"), "-o", "abi.o"], d)
    _run(["g++"] + SAN + ["-o", "drv", "drv.o", "abi.o"] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], d)
    return os.path.join(d, "drv")


def test_abi_host_code_is_sanitizer_clean(driver):
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations; leaks are not what is checked here
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HIP_VISIBLE_DEVICES"] = ""                 # never a device, even where one exists
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert ", 0 failures" in r.stdout
