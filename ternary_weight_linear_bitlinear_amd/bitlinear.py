"""Thin Python binding of ``libbitlinear.so`` (the C ABI in include/bitlinear.h).

Argument marshalling only: torch provides device memory and the current
stream; every step of the BitLinear pass runs in the library's HIP kernels.
There is no CPU or PyTorch fallback: if the library is missing, importing
this module raises.

Functions keep the C names (``bitlinear_pack_weights``,
``bitlinear_quant_acts``, ``bitlinear_forward``, ``bitlinear_linear``,
``bitlinear_backward_input``, ``bitlinear_backward_weight``) and take torch
tensors; ``linear`` chains activation quantisation and the forward product.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitlinear.so")

BL_OK, BL_ERR_INVALID_ARG, BL_ERR_UNSUPPORTED, BL_ERR_DEVICE = 0, 1, 2, 3
BL_F32, BL_BF16 = 0, 1
BL_PACK_2BIT, BL_PACK_BASE3, BL_PACK_1BIT = 0, 1, 2
BL_TERNARY, BL_BINARY = 0, 1

LAYOUTS = {"2bit": BL_PACK_2BIT, "base3": BL_PACK_BASE3, "1bit": BL_PACK_1BIT}
SCHEMES = {"ternary": BL_TERNARY, "binary": BL_BINARY}
_DTYPES = {torch.float32: BL_F32, torch.bfloat16: BL_BF16}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m ternary_weight_linear_bitlinear_amd.build` "
        "(there is no fallback path)")

_lib = ctypes.CDLL(LIB_PATH)
_lib.bitlinear_source_hash.restype = ctypes.c_char_p
_lib.bitlinear_source_hash.argtypes = []


def _refuse_stale_library() -> None:
    """A library built from other sources than the ones beside it would be
    tested and timed in their place: refuse it."""
    from . import build as _build
    if not os.path.isdir(_build.CSRC):
        return  # an installed library without its sources: nothing to compare
    built = _lib.bitlinear_source_hash().decode()
    here = _build.source_hash()
    if built != here:
        raise ImportError(
            f"{LIB_PATH} was built from other sources (library {built}, sources {here}): rebuild "
            "it with `python -m ternary_weight_linear_bitlinear_amd.build`")


_refuse_stale_library()
_p, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_lib.bitlinear_packed_row_bytes.restype = _i64
_lib.bitlinear_packed_row_bytes.argtypes = [_i64, _int]
_lib.bitlinear_pack_workspace_bytes.restype = _sz
_lib.bitlinear_pack_workspace_bytes.argtypes = [_i64, _i64]
_lib.bitlinear_pack_weights.restype = _int
_lib.bitlinear_pack_weights.argtypes = [_p, _int, _i64, _i64, _int, _int, _f32, _p, _p, _p, _sz, _p]
_lib.bitlinear_pack_weights_noalloc.restype = _int
_lib.bitlinear_pack_weights_noalloc.argtypes = [_p, _int, _i64, _i64, _int, _int, _f32, _p, _p, _p]
_lib.bitlinear_pack_noalloc_max_scratch_bytes.restype = _sz
_lib.bitlinear_pack_noalloc_max_scratch_bytes.argtypes = []
_lib.bitlinear_quant_acts.restype = _int
_lib.bitlinear_quant_acts.argtypes = [_p, _int, _i64, _i64, _p, _p, _p]
_lib.bitlinear_forward.restype = _int
_lib.bitlinear_forward.argtypes = [_p, _p, _p, _int, _p, _i64, _i64, _i64, _p, _int, _p, _p]
_lib.bitlinear_linear.restype = _int
_lib.bitlinear_linear.argtypes = [_p, _int, _p, _int, _p, _i64, _i64, _i64, _p, _int, _p, _p]
_lib.bitlinear_forward_segmented.restype = _int
_lib.bitlinear_forward_segmented.argtypes = [_p, _p, _p, _int, _p, _p, _int, _i64, _i64, _p, _int,
                                             _p, _p]
_lib.bitlinear_linear_segmented.restype = _int
_lib.bitlinear_linear_segmented.argtypes = [_p, _int, _p, _int, _p, _p, _int, _i64, _i64, _p, _int,
                                            _p, _p]
_lib.bitlinear_forward_lut.restype = _int
_lib.bitlinear_forward_lut.argtypes = [_p, _p, _p, _int, _p, _i64, _i64, _i64, _p, _int, _p, _p]
_lib.bitlinear_backward_input.restype = _int
_lib.bitlinear_backward_input.argtypes = [_p, _int, _p, _int, _p, _i64, _i64, _i64, _p, _p]
_lib.bitlinear_backward_weight.restype = _int
_lib.bitlinear_backward_weight.argtypes = [_p, _p, _int, _i64, _i64, _i64, _p, _p]
_lib.bitlinear_forward_plan.restype = _int
_lib.bitlinear_forward_plan.argtypes = [_i64, _i64, _i64, _int, _int, _int, ctypes.c_char_p, _sz]
_lib.bitlinear_status_string.restype = ctypes.c_char_p
_lib.bitlinear_status_string.argtypes = [_int]
_lib.bitlinear_version.restype = _int
_lib.bitlinear_version.argtypes = []

EXPORTED = ["bitlinear_packed_row_bytes", "bitlinear_pack_workspace_bytes",
            "bitlinear_pack_weights", "bitlinear_pack_weights_noalloc",
            "bitlinear_pack_noalloc_max_scratch_bytes", "bitlinear_quant_acts", "bitlinear_forward",
            "bitlinear_linear", "bitlinear_forward_segmented", "bitlinear_linear_segmented",
            "bitlinear_forward_lut", "bitlinear_backward_input", "bitlinear_backward_weight",
            "bitlinear_forward_plan", "bitlinear_status_string", "bitlinear_version",
            "bitlinear_source_hash"]
FUSED_MAX_M = 4


class BitLinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.bitlinear_status_string(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != BL_OK:
        raise BitLinearError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _layout(layout) -> int:
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def library() -> ctypes.CDLL:
    return _lib


# ----------------------------------------------------------------------------
def bitlinear_packed_row_bytes(K: int, layout="2bit") -> int:
    return int(_lib.bitlinear_packed_row_bytes(K, _layout(layout)))


def bitlinear_pack_workspace_bytes(N: int, K: int) -> int:
    return int(_lib.bitlinear_pack_workspace_bytes(N, K))


def bitlinear_version() -> int:
    return int(_lib.bitlinear_version())


def bitlinear_forward_plan(M: int, N: int, K: int, layout="2bit", out_dtype=torch.float32,
                           fused: bool = False) -> list[str]:
    """The kernel launches bitlinear_forward (or, with fused=True,
    bitlinear_linear on bf16 x) would make for an M x N x K product, one
    string per launch; nothing is launched."""
    buf = ctypes.create_string_buffer(8192)
    n = _lib.bitlinear_forward_plan(M, N, K, _layout(layout), _DTYPES[out_dtype], int(fused),
                                    buf, len(buf))
    if n < 0:
        raise BitLinearError(BL_ERR_INVALID_ARG, "bitlinear_forward_plan")
    lines = buf.value.decode().splitlines()
    assert len(lines) == n
    return lines


def bitlinear_status_string(status: int) -> str:
    return _lib.bitlinear_status_string(status).decode()


def bitlinear_pack_weights(W: torch.Tensor, layout="2bit", scheme="ternary", eps: float = 1e-5,
                           packed: torch.Tensor | None = None, gamma: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None):
    """Quantise and pack W [N, K] (fp32 or bf16, on the GPU).

    Returns (packed uint8 [N, row_bytes], gamma float32 [1]) on W's device."""
    assert W.dim() == 2 and W.is_contiguous() and W.dtype in _DTYPES
    N, K = W.shape
    lay = _layout(layout)
    rb = bitlinear_packed_row_bytes(K, lay)
    dev = W.device
    if packed is None:
        packed = torch.empty((N, rb), dtype=torch.uint8, device=dev)
    if gamma is None:
        gamma = torch.empty(4, dtype=torch.float32, device=dev)[:1]
    wsb = bitlinear_pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _check(_lib.bitlinear_pack_weights(_ptr(W), _DTYPES[W.dtype], N, K,
                                       SCHEMES[scheme] if isinstance(scheme, str) else int(scheme),
                                       lay, float(eps), _ptr(packed), _ptr(gamma),
                                       _ptr(workspace), workspace.numel(), _stream(stream)),
           "bitlinear_pack_weights")
    return packed, gamma


def bitlinear_pack_weights_noalloc(W: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor,
                                   layout="2bit", scheme="ternary", eps: float = 1e-5,
                                   stream=None):
    """bitlinear_pack_weights into caller-provided packed / gamma, with the
    library's own scratch instead of a workspace (nothing is allocated)."""
    assert W.dim() == 2 and W.is_contiguous() and W.dtype in _DTYPES
    N, K = W.shape
    _check(_lib.bitlinear_pack_weights_noalloc(
        _ptr(W), _DTYPES[W.dtype], N, K, SCHEMES[scheme] if isinstance(scheme, str) else int(scheme),
        _layout(layout), float(eps), _ptr(packed), _ptr(gamma), _stream(stream)),
        "bitlinear_pack_weights_noalloc")
    return packed, gamma


def bitlinear_pack_noalloc_max_scratch_bytes() -> int:
    return int(_lib.bitlinear_pack_noalloc_max_scratch_bytes())


def bitlinear_quant_acts(x: torch.Tensor, xq: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None, stream=None):
    """Per-token INT8 quantisation of x [M, K]; returns (xq int8 [M, K], scale f32 [M])."""
    assert x.dim() == 2 and x.is_contiguous() and x.dtype in _DTYPES
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty(max(M, 1), dtype=torch.float32, device=x.device)[:M]
    _check(_lib.bitlinear_quant_acts(_ptr(x), _DTYPES[x.dtype], M, K, _ptr(xq), _ptr(scale),
                                     _stream(stream)), "bitlinear_quant_acts")
    return xq, scale


def bitlinear_forward(xq: torch.Tensor, scale: torch.Tensor, packed: torch.Tensor,
                      gamma: torch.Tensor, N: int, K: int, layout="2bit",
                      out_dtype=torch.float32, y: torch.Tensor | None = None,
                      acc: torch.Tensor | bool | None = None, stream=None):
    """y = (xq c^T) * gamma * scale / 127; returns y, or (y, acc) when acc is requested."""
    M = xq.shape[0]
    assert xq.dim() == 2 and xq.shape[1] == K and xq.dtype == torch.int8
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    want_acc = acc is not None and acc is not False
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _check(_lib.bitlinear_forward(_ptr(xq), _ptr(scale), _ptr(packed), _layout(layout),
                                  _ptr(gamma), M, N, K, _ptr(y), _DTYPES[y.dtype],
                                  _ptr(acc) if want_acc else None, _stream(stream)),
           "bitlinear_forward")
    return (y, acc) if want_acc else y


def bitlinear_linear(x: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, N: int,
                     layout="2bit", out_dtype=torch.float32, y: torch.Tensor | None = None,
                     acc: torch.Tensor | bool | None = None, stream=None):
    """Fused quantise + multiply for M <= 4 tokens; returns y, or (y, acc)."""
    assert x.dim() == 2 and x.is_contiguous() and x.dtype in _DTYPES
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    want_acc = acc is not None and acc is not False
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=x.device)
    _check(_lib.bitlinear_linear(_ptr(x), _DTYPES[x.dtype], _ptr(packed), _layout(layout),
                                 _ptr(gamma), M, N, K, _ptr(y), _DTYPES[y.dtype],
                                 _ptr(acc) if want_acc else None, _stream(stream)),
           "bitlinear_linear")
    return (y, acc) if want_acc else y


def bitlinear_forward_lut(xq: torch.Tensor, scale: torch.Tensor, packed: torch.Tensor,
                          gamma: torch.Tensor, N: int, K: int, out_dtype=torch.float32,
                          y: torch.Tensor | None = None, acc: torch.Tensor | bool | None = None,
                          stream=None):
    """One token against base-3 codes through activation-side lookup tables."""
    M = xq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    want_acc = acc is not None and acc is not False
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _check(_lib.bitlinear_forward_lut(_ptr(xq), _ptr(scale), _ptr(packed), BL_PACK_BASE3,
                                      _ptr(gamma), M, N, K, _ptr(y), _DTYPES[y.dtype],
                                      _ptr(acc) if want_acc else None, _stream(stream)),
           "bitlinear_forward_lut")
    return (y, acc) if want_acc else y


def _seg_table(seg_rows):
    rows = [int(r) for r in seg_rows]
    return (ctypes.c_int64 * len(rows))(*rows), len(rows), sum(rows)


def bitlinear_forward_segmented(xq: torch.Tensor, scale: torch.Tensor, packed: torch.Tensor,
                                gammas: torch.Tensor, seg_rows, K: int, layout="2bit",
                                out_dtype=torch.float32, y: torch.Tensor | None = None,
                                acc: torch.Tensor | bool | None = None, stream=None):
    """bitlinear_forward over a stack of row segments, each with its own gamma
    (gammas[s]); y [M, sum(seg_rows)]."""
    M = xq.shape[0]
    table, nseg, N = _seg_table(seg_rows)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    want_acc = acc is not None and acc is not False
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _check(_lib.bitlinear_forward_segmented(_ptr(xq), _ptr(scale), _ptr(packed), _layout(layout),
                                            _ptr(gammas), table, nseg, M, K, _ptr(y),
                                            _DTYPES[y.dtype], _ptr(acc) if want_acc else None,
                                            _stream(stream)), "bitlinear_forward_segmented")
    return (y, acc) if want_acc else y


def bitlinear_linear_segmented(x: torch.Tensor, packed: torch.Tensor, gammas: torch.Tensor,
                               seg_rows, layout="2bit", out_dtype=torch.float32,
                               y: torch.Tensor | None = None,
                               acc: torch.Tensor | bool | None = None, stream=None):
    """Fused quantise + multiply (M <= 4) over a stack of row segments."""
    assert x.dim() == 2 and x.is_contiguous() and x.dtype in _DTYPES
    M, K = x.shape
    table, nseg, N = _seg_table(seg_rows)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    want_acc = acc is not None and acc is not False
    if acc is True:
        acc = torch.empty((M, N), dtype=torch.int32, device=x.device)
    _check(_lib.bitlinear_linear_segmented(_ptr(x), _DTYPES[x.dtype], _ptr(packed),
                                           _layout(layout), _ptr(gammas), table, nseg, M, K,
                                           _ptr(y), _DTYPES[y.dtype],
                                           _ptr(acc) if want_acc else None, _stream(stream)),
           "bitlinear_linear_segmented")
    return (y, acc) if want_acc else y


def bitlinear_backward_input(grad_y: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor,
                             K: int, layout="2bit", grad_x: torch.Tensor | None = None,
                             stream=None) -> torch.Tensor:
    """grad_x [M, K] fp32 = gamma * grad_y [M, N] (bf16) x codes of packed [N, row_bytes]."""
    assert grad_y.dim() == 2 and grad_y.is_contiguous() and grad_y.dtype in _DTYPES
    M, N = grad_y.shape
    if grad_x is None:
        grad_x = torch.empty((M, K), dtype=torch.float32, device=grad_y.device)
    _check(_lib.bitlinear_backward_input(_ptr(grad_y), _DTYPES[grad_y.dtype], _ptr(packed),
                                         _layout(layout), _ptr(gamma), M, N, K, _ptr(grad_x),
                                         _stream(stream)), "bitlinear_backward_input")
    return grad_x


def bitlinear_backward_weight(grad_y: torch.Tensor, x: torch.Tensor,
                              grad_w: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """grad_w [N, K] fp32 = grad_y^T (bf16 [M, N]) x x (bf16 [M, K])."""
    assert grad_y.dim() == 2 and x.dim() == 2 and grad_y.shape[0] == x.shape[0]
    assert grad_y.is_contiguous() and x.is_contiguous() and grad_y.dtype == x.dtype
    M, N = grad_y.shape
    K = x.shape[1]
    if grad_w is None:
        grad_w = torch.empty((N, K), dtype=torch.float32, device=x.device)
    _check(_lib.bitlinear_backward_weight(_ptr(grad_y), _ptr(x), _DTYPES[x.dtype], M, N, K,
                                          _ptr(grad_w), _stream(stream)),
           "bitlinear_backward_weight")
    return grad_w


def linear(x: torch.Tensor, packed: torch.Tensor, gamma: torch.Tensor, N: int, layout="2bit",
           out_dtype=torch.float32, stream=None) -> torch.Tensor:
    """BitLinear forward of x [M, K] against packed weights: one fused launch for
    M <= 4, otherwise quantise then multiply."""
    if x.shape[0] <= FUSED_MAX_M:
        return bitlinear_linear(x, packed, gamma, N, layout, out_dtype, stream=stream)
    xq, scale = bitlinear_quant_acts(x, stream=stream)
    return bitlinear_forward(xq, scale, packed, gamma, N, x.shape[1], layout, out_dtype,
                             stream=stream)
