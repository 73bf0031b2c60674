"""Build the HIP library ``libbitlinear.so`` for gfx950 with hipcc.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then all are linked into ``libbitlinear.so`` next to this file.
Run as ``python -m ternary_weight_linear_bitlinear_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libbitlinear.so")
# measurement probes for the benchmark (stream read, empty launch, INT8
# matrix-core loop); a separate library, not part of the BitLinear ABI
PROBES_SRC = os.path.join(PKG, "probes", "probes.hip")
PROBES_PATH = os.path.join(PKG, "libblprobes.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def source_files() -> list[str]:
    """Every file the library is built from: csrc/*.hip, csrc/*.hpp and the
    public header."""
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
                  + [os.path.join(INCLUDE, "bitlinear.h")])


def source_hash() -> str:
    """SHA-256 (first 32 hex digits) over the names and contents of
    source_files(); compiled into the library, so the binding can refuse a
    library built from other sources."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:32]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return path


def _compile(src: str, digest: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, f'-DBL_SOURCE_HASH="{digest}"', "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    digest = source_hash()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, digest), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    build_probes(verbose)
    return LIB_PATH


def build_probes(verbose: bool = False) -> str:
    tmp = PROBES_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", PROBES_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBES_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBES_PATH)
    if verbose:
        print(f"built {PROBES_PATH}")
    return PROBES_PATH


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
