"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer.

- The oracle (plain C, gcc) under a driver that runs every oracle function over
  ragged shapes (tests/sanitize/oracle_driver.c).
- The library's host code (hipcc, sanitizers on the host pass only: device code
  is built as usual) under a driver that runs argument validation, the size
  helpers and the dispatch's dry run over valid, invalid and extreme shapes
  (tests/sanitize/abi_driver.c). Without a GPU, valid calls stop at the device
  check. The build is cached under _build/sanitize, keyed by the sources.

Either driver fails on a sanitizer finding (errors are not recoverable) or on
an unexpected status.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from ternary_weight_linear_bitlinear_amd import build as B  # noqa: E402

HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_sanitizers():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp",
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "bitlinear_oracle.c"),
         "-o", exe, "-lm"])
    r = run([exe], env=ENV, timeout=300)
    assert "oracle driver: ok" in r.stdout


def _build_abi_driver() -> str:
    digest = B.source_hash()
    exe = os.path.join(OUT, f"abi_driver_{digest}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT, exist_ok=True)
    for old in os.listdir(OUT):  # drivers of older sources
        if old.startswith("abi_driver_"):
            os.remove(os.path.join(OUT, old))
    hipcc = B.hipcc()
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    procs = []
    for name in sorted(os.listdir(B.CSRC)):
        if not name.endswith(".hip"):
            continue
        obj = os.path.join(OUT, name + ".o")
        objs.append(obj)
        cmd = [hipcc, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *host_san,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", B.INCLUDE, "-I", B.CSRC, f'-DBL_SOURCE_HASH="{digest}"',
               "-c", os.path.join(B.CSRC, name), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    for cmd, p in procs:
        out, err = p.communicate(timeout=900)
        assert p.returncode == 0, f"{' '.join(cmd)}\n{err[-3000:]}"
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    drv = os.path.join(OUT, "abi_driver.o")
    run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", B.INCLUDE, "-c", os.path.join(HERE, "abi_driver.c"), "-o", drv])
    tmp = exe + ".tmp"
    run([hipcc, f"--offload-arch={B.ARCH}", *host_san, drv, *objs, "-o", tmp])
    os.replace(tmp, exe)
    return exe


def test_abi_host_code_under_sanitizers():
    exe = _build_abi_driver()
    import torch
    args = [exe] + (["gpu"] if torch.cuda.is_available() else [])
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")  # the HIP runtime keeps its own allocations
    r = run(args, env=env, timeout=300)
    assert "abi driver: ok" in r.stdout
