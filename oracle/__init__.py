"""Python wrapper around the C oracle (``bitlinear_oracle.c``).

THIS IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the
HIP library and its Python binding) never imports, loads or calls anything
here, and nothing here imports the product.

The wrapper only marshals numpy arrays into the C functions; every step of
the method runs in the C file, which cites the pages it follows. All
functions take float32 inputs (bf16 inputs are widened exactly by the
caller) and return numpy arrays.

Parity pins live in ``tests/test_oracle_pins.py``. Every function here is
pinned there (none is "parity unpinned").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
LIB_PATH = os.path.join(_HERE, "liborcl.so")

GCC_CMD = [
    "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
    "-fPIC", "-shared", _SRC, "-o", LIB_PATH, "-lm",
]


def build() -> str:
    """Compile the oracle shared library with gcc (plain scalar C, -O2)."""
    subprocess.run(GCC_CMD, check=True)
    return LIB_PATH


_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "orc_absmean": (ctypes.c_float, [_p, _i64, _p]),
        "orc_mean": (ctypes.c_float, [_p, _i64, _p]),
        "orc_ternary_codes": (_i64, [_p, _i64, ctypes.c_float, ctypes.c_float, ctypes.c_double, _p, _p]),
        "orc_binary_codes": (_i64, [_p, _i64, ctypes.c_float, ctypes.c_double, _p, _p]),
        "orc_row_bytes_2bit": (_i64, [_i64]),
        "orc_pack_2bit": (None, [_p, _i64, _i64, _p]),
        "orc_unpack_2bit": (_i64, [_p, _i64, _i64, _p]),
        "orc_row_bytes_base3": (_i64, [_i64]),
        "orc_pack_base3": (None, [_p, _i64, _i64, _p]),
        "orc_unpack_base3": (_i64, [_p, _i64, _i64, _p]),
        "orc_row_bytes_1bit": (_i64, [_i64]),
        "orc_pack_1bit": (_i64, [_p, _i64, _i64, _p]),
        "orc_unpack_1bit": (_i64, [_p, _i64, _i64, _p]),
        "orc_quant_acts": (_i64, [_p, _i64, _i64, _p, _p, _p]),
        "orc_int_product": (_i64, [_p, _p, _i64, _i64, _i64, _p]),
        "orc_epilogue": (None, [_p, ctypes.c_float, _p, _i64, _i64, _p]),
        "orc_bf16_rne_array": (None, [_p, _i64, _p]),
        "orc_ste_grad_x": (None, [_p, _p, ctypes.c_float, _i64, _i64, _i64, _p]),
        "orc_ste_grad_w": (None, [_p, _p, _i64, _i64, _i64, _p]),
        "orc_num_threads": (ctypes.c_int, []),
        "orc_set_num_threads": (None, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
def absmean(w: np.ndarray) -> tuple[np.float32, float]:
    """gamma = mean|W| (fp64 accumulate, rounded once); returns (fp32, fp64)."""
    w = _c(w, np.float32)
    m64 = ctypes.c_double()
    g = _load().orc_absmean(_ptr(w), w.size, ctypes.byref(m64))
    return np.float32(g), m64.value


def mean(w: np.ndarray) -> tuple[np.float32, float]:
    """alpha = mean(W) for the 1-bit variant; returns (fp32, fp64)."""
    w = _c(w, np.float32)
    m64 = ctypes.c_double()
    a = _load().orc_mean(_ptr(w), w.size, ctypes.byref(m64))
    return np.float32(a), m64.value


def ternary_codes(w: np.ndarray, eps: float = 1e-5, gamma=None):
    """Ternary codes of W (same shape, int8) and boundary flags (uint8).

    gamma defaults to the oracle's own absmean. Returns (codes, flags, gamma32).
    """
    w = _c(w, np.float32)
    if gamma is None:
        g32, g64 = absmean(w)
    else:
        g32, g64 = np.float32(gamma), float(np.float32(gamma))
    codes = np.empty(w.shape, np.int8)
    flags = np.empty(w.shape, np.uint8)
    _load().orc_ternary_codes(_ptr(w), w.size, float(g32), float(np.float32(eps)), g64,
                              _ptr(codes), _ptr(flags))
    return codes, flags, g32


def binary_codes(w: np.ndarray):
    """1-bit codes (+1 above the mean alpha, else -1), flags and (alpha, beta).

    beta = mean|W| is the weight scale of the 1-bit variant.
    """
    w = _c(w, np.float32)
    a32, a64 = mean(w)
    b32, _ = absmean(w)
    codes = np.empty(w.shape, np.int8)
    flags = np.empty(w.shape, np.uint8)
    _load().orc_binary_codes(_ptr(w), w.size, float(a32), a64, _ptr(codes), _ptr(flags))
    return codes, flags, a32, b32


def row_bytes(K: int, layout: str) -> int:
    lib = _load()
    if layout == "2bit":
        return int(lib.orc_row_bytes_2bit(K))
    if layout == "base3":
        return int(lib.orc_row_bytes_base3(K))
    if layout == "1bit":
        return int(lib.orc_row_bytes_1bit(K))
    raise ValueError(layout)


def _layout_fns(layout: str):
    lib = _load()
    return {"2bit": (lib.orc_pack_2bit, lib.orc_unpack_2bit),
            "base3": (lib.orc_pack_base3, lib.orc_unpack_base3),
            "1bit": (lib.orc_pack_1bit, lib.orc_unpack_1bit)}[layout]


def pack(codes: np.ndarray, layout: str) -> np.ndarray:
    """Pack int8 codes [N, K] into the canonical layout [N, row_bytes]. The
    1-bit layout holds +-1 codes only (ValueError otherwise)."""
    codes = _c(codes, np.int8)
    N, K = codes.shape
    out = np.empty((N, row_bytes(K, layout)), np.uint8)
    bad = _layout_fns(layout)[0](_ptr(codes), N, K, _ptr(out))
    if layout == "1bit" and bad:
        raise ValueError(f"{bad} codes are not +-1: no 1-bit encoding")
    return out


def unpack(packed: np.ndarray, K: int, layout: str) -> tuple[np.ndarray, int]:
    """Inverse of pack for k < K; returns (codes, number of invalid fields)."""
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] == row_bytes(K, layout)
    codes = np.empty((N, K), np.int8)
    bad = _layout_fns(layout)[1](_ptr(packed), N, K, _ptr(codes))
    return codes, int(bad)


def quant_acts(x: np.ndarray):
    """Per-token absmax INT8 codes [M, K], scales [M] and boundary flags."""
    x = _c(x, np.float32)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    scale = np.empty(M, np.float32)
    flags = np.empty((M, K), np.uint8)
    _load().orc_quant_acts(_ptr(x), M, K, _ptr(xq), _ptr(scale), _ptr(flags))
    return xq, scale, flags


def int_product(xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k xq[m, k] * codes[n, k] as int32 (brute force)."""
    xq = _c(xq, np.int8)
    codes = _c(codes, np.int8)
    M, K = xq.shape
    N, K2 = codes.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    ovf = _load().orc_int_product(_ptr(xq), _ptr(codes), M, N, K, _ptr(acc))
    if ovf:
        raise OverflowError(f"{ovf} accumulators exceed int32")
    return acc


def epilogue(acc: np.ndarray, gamma, scale: np.ndarray) -> np.ndarray:
    """y = acc * gamma * scale[m] / 127 in fp64 (unrounded)."""
    acc = _c(acc, np.int32)
    scale = _c(scale, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _load().orc_epilogue(_ptr(acc), float(np.float32(gamma)), _ptr(scale), M, N, _ptr(y))
    return y


def bf16_rne(f: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().orc_bf16_rne_array(_ptr(f), f.size, _ptr(out))
    return out


def ste_grad_x(grad_y: np.ndarray, codes: np.ndarray, gamma) -> np.ndarray:
    grad_y = _c(grad_y, np.float32)
    codes = _c(codes, np.int8)
    M, N = grad_y.shape
    N2, K = codes.shape
    assert N == N2
    out = np.empty((M, K), np.float64)
    _load().orc_ste_grad_x(_ptr(grad_y), _ptr(codes), float(np.float32(gamma)), M, N, K, _ptr(out))
    return out


def ste_grad_w(grad_y: np.ndarray, x: np.ndarray) -> np.ndarray:
    grad_y = _c(grad_y, np.float32)
    x = _c(x, np.float32)
    M, N = grad_y.shape
    M2, K = x.shape
    assert M == M2
    out = np.empty((N, K), np.float64)
    _load().orc_ste_grad_w(_ptr(grad_y), _ptr(x), M, N, K, _ptr(out))
    return out


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on."""
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------
def forward(w: np.ndarray, x: np.ndarray, layout: str = "2bit", scheme: str = "ternary",
            eps: float = 1e-5) -> dict:
    """The whole BitLinear forward on fp32 (or exactly widened bf16) inputs.

    Returns every intermediate: gamma, codes, packed bytes, activation codes and
    scales, boundary flags, the int32 accumulators and the fp64 output.
    """
    if scheme == "ternary":
        codes, wflags, gamma = ternary_codes(w, eps)
    elif scheme == "binary":
        codes, wflags, _alpha, gamma = binary_codes(w)
    else:
        raise ValueError(scheme)
    packed = pack(codes, layout)
    xq, scale, xflags = quant_acts(x)
    acc = int_product(xq, codes)
    y64 = epilogue(acc, gamma, scale)
    return dict(gamma=gamma, codes=codes, wflags=wflags, packed=packed, xq=xq,
                scale=scale, xflags=xflags, acc=acc, y64=y64)
