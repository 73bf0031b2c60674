"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/bitlinear.h declares, computes the pure size helpers,
and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


@pytest.fixture(scope="module")
def bl():
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_header_symbols_exported(bl):
    names = declared_functions()
    assert len(names) >= 7
    lib = bl.library()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bl.EXPORTED) == names


def test_status_strings_and_version(bl):
    assert bl.bitlinear_status_string(0) == "ok"
    assert "invalid" in bl.bitlinear_status_string(1)
    assert bl.bitlinear_version() >> 16 == 1


def test_row_bytes(bl):
    import oracle
    for K in [1, 3, 4, 5, 16, 63, 64, 65, 79, 80, 81, 4096, 11008]:
        assert bl.bitlinear_packed_row_bytes(K, "2bit") == oracle.row_bytes(K, "2bit")
        assert bl.bitlinear_packed_row_bytes(K, "base3") == oracle.row_bytes(K, "base3")
        assert bl.bitlinear_packed_row_bytes(K, "1bit") == oracle.row_bytes(K, "1bit")
    assert bl.bitlinear_packed_row_bytes(0, "2bit") == -1
    assert bl.bitlinear_packed_row_bytes(16, 7) == -1
    assert bl.bitlinear_packed_row_bytes(4096, "2bit") == 1024
    assert bl.bitlinear_packed_row_bytes(4096, "base3") == 832
    assert bl.bitlinear_packed_row_bytes(4096, "1bit") == 512
    assert bl.bitlinear_pack_workspace_bytes(0, 5) == 0
    assert bl.bitlinear_pack_workspace_bytes(4096, 4096) % 16 == 0
    assert bl.bitlinear_pack_workspace_bytes(1 << 40, 1 << 30) == 0  # N * K past int64


P = 0x10000  # a fake, 16-byte aligned address: never dereferenced on these paths


def _pack(bl, **kw):
    a = dict(W=P, dt=0, N=4, K=64, scheme=0, layout=0, eps=1e-5, packed=P, gamma=P, ws=P,
             wsb=1 << 20, stream=None)
    a.update(kw)
    return bl.library().bitlinear_pack_weights(a["W"], a["dt"], a["N"], a["K"], a["scheme"],
                                                a["layout"], a["eps"], a["packed"], a["gamma"],
                                                a["ws"], a["wsb"], a["stream"])


def _quant(bl, **kw):
    a = dict(x=P, dt=0, M=4, K=64, xq=P, scale=P, stream=None)
    a.update(kw)
    return bl.library().bitlinear_quant_acts(a["x"], a["dt"], a["M"], a["K"], a["xq"],
                                              a["scale"], a["stream"])


def _fwd(bl, **kw):
    a = dict(xq=P, scale=P, packed=P, layout=0, gamma=P, M=4, N=8, K=64, y=P, ydt=0, acc=None,
             stream=None)
    a.update(kw)
    return bl.library().bitlinear_forward(a["xq"], a["scale"], a["packed"], a["layout"],
                                          a["gamma"], a["M"], a["N"], a["K"], a["y"], a["ydt"],
                                          a["acc"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(W=None), dict(packed=None), dict(gamma=None), dict(ws=None), dict(W=P + 4),
    dict(gamma=P + 2),
    dict(packed=P + 8), dict(N=0), dict(N=-1), dict(K=0), dict(K=16909321), dict(dt=2),
    dict(scheme=5), dict(layout=3), dict(eps=-1.0), dict(eps=float("nan")), dict(wsb=0),
    dict(layout=2, scheme=0),  # the 1-bit layout holds binary codes only
])
def test_pack_rejects(bl, kw):
    assert _pack(bl, **kw) == bl.BL_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(xq=None), dict(scale=None), dict(x=P + 2), dict(M=-1), dict(K=0),
    dict(K=16909321), dict(dt=9),
])
def test_quant_rejects(bl, kw):
    assert _quant(bl, **kw) == bl.BL_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [
    dict(xq=None), dict(scale=None), dict(packed=None), dict(gamma=None), dict(y=None),
    dict(gamma=P + 1),
    dict(y=P + 4), dict(acc=P + 4), dict(M=-1), dict(N=-1), dict(K=0), dict(K=16909321),
    dict(layout=3), dict(ydt=3),
])
def test_forward_rejects(bl, kw):
    assert _fwd(bl, **kw) == bl.BL_ERR_INVALID_ARG


def test_empty_problems_are_noops(bl):
    assert _quant(bl, M=0) == bl.BL_OK
    assert _fwd(bl, M=0) == bl.BL_OK
    assert _fwd(bl, N=0) == bl.BL_OK


def test_no_device_reports_device_error(bl):
    """Valid arguments with no gfx950 device visible: BL_ERR_DEVICE, nothing launched."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _pack(bl) == bl.BL_ERR_DEVICE
    assert _quant(bl) == bl.BL_ERR_DEVICE
    assert _fwd(bl) == bl.BL_ERR_DEVICE


def test_fused_linear_rejects_and_limits(bl):
    lib = bl.library()
    f = lambda **kw: lib.bitlinear_linear(kw.get("x", P), 0, P, kw.get("layout", 0), P,
                                          kw.get("M", 1), 8, kw.get("K", 64), kw.get("y", P), 0,
                                          None, None)
    assert f(x=None) == bl.BL_ERR_INVALID_ARG
    assert f(y=P + 4) == bl.BL_ERR_INVALID_ARG
    assert f(K=0) == bl.BL_ERR_INVALID_ARG
    assert f(layout=9) == bl.BL_ERR_INVALID_ARG
    assert f(M=5) == bl.BL_ERR_UNSUPPORTED  # fused path covers M <= 4 only
    assert f(M=0) == bl.BL_OK


def test_backward_rejects_and_limits(bl):
    lib = bl.library()
    bi = lambda **kw: lib.bitlinear_backward_input(kw.get("gy", P), kw.get("dt", 1), P,
                                                   kw.get("layout", 0), kw.get("gamma", P),
                                                   kw.get("M", 4), kw.get("N", 64),
                                                   kw.get("K", 64), kw.get("gx", P), None)
    assert bi(gy=None) == bl.BL_ERR_INVALID_ARG
    assert bi(gamma=None) == bl.BL_ERR_INVALID_ARG
    assert bi(gamma=P + 2) == bl.BL_ERR_INVALID_ARG
    assert bi(gx=P + 4) == bl.BL_ERR_INVALID_ARG
    assert bi(K=0) == bl.BL_ERR_INVALID_ARG
    assert bi(M=-1) == bl.BL_ERR_INVALID_ARG
    assert bi(N=(1 << 24) + 8) == bl.BL_ERR_INVALID_ARG
    assert bi(dt=5) == bl.BL_ERR_INVALID_ARG
    assert bi(layout=4) == bl.BL_ERR_INVALID_ARG
    assert bi(N=60) == bl.BL_ERR_UNSUPPORTED       # N % 8 != 0
    assert bi(layout=1, dt=0, N=4) == bl.BL_ERR_UNSUPPORTED
    assert bi(layout=2, N=60) == bl.BL_ERR_UNSUPPORTED
    assert bi(M=0) == bl.BL_OK
    bw = lambda **kw: lib.bitlinear_backward_weight(kw.get("gy", P), kw.get("x", P),
                                                    kw.get("dt", 1), kw.get("M", 4),
                                                    kw.get("N", 64), kw.get("K", 64),
                                                    kw.get("gw", P), None)
    assert bw(x=None) == bl.BL_ERR_INVALID_ARG
    assert bw(gw=P + 8) == bl.BL_ERR_INVALID_ARG
    assert bw(K=0) == bl.BL_ERR_INVALID_ARG
    assert bw(dt=3) == bl.BL_ERR_INVALID_ARG
    assert bw(dt=0, K=60) == bl.BL_ERR_UNSUPPORTED
    assert bw(K=60) == bl.BL_ERR_UNSUPPORTED
    assert bw(N=12) == bl.BL_ERR_UNSUPPORTED
    assert bw(N=0) == bl.BL_OK
    import torch
    if not torch.cuda.is_available():
        assert bi() == bl.BL_ERR_DEVICE
        assert bw() == bl.BL_ERR_DEVICE


def test_segmented_rejects(bl):
    import ctypes
    lib = bl.library()
    T = lambda *r: (ctypes.c_int64 * len(r))(*r)

    def fs(table, nseg, **kw):
        return lib.bitlinear_forward_segmented(P, P, P, kw.get("layout", 0), kw.get("g", P), table,
                                               nseg, kw.get("M", 4), 64, P, 0, None, None)

    def ls(table, nseg, **kw):
        return lib.bitlinear_linear_segmented(P, 0, P, 0, kw.get("g", P), table, nseg,
                                              kw.get("M", 1), 64, P, 0, None, None)
    for f in (fs, ls):
        assert f(None, 2) == bl.BL_ERR_INVALID_ARG
        assert f(T(16, 16), 0) == bl.BL_ERR_INVALID_ARG
        assert f(T(*([16] * 9)), 9) == bl.BL_ERR_INVALID_ARG
        assert f(T(16, 0, 16), 3) == bl.BL_ERR_INVALID_ARG
        assert f(T(16, -4), 2) == bl.BL_ERR_INVALID_ARG
        assert f(T(16, 16), 2, g=None) == bl.BL_ERR_INVALID_ARG
        assert f(T(16, 16), 2, g=P + 2) == bl.BL_ERR_INVALID_ARG
        assert f(T(16, 16), 2, M=0) == bl.BL_OK
    assert ls(T(16, 16), 2, M=5) == bl.BL_ERR_UNSUPPORTED
    import torch
    if not torch.cuda.is_available():
        assert fs(T(16, 16), 2) == bl.BL_ERR_DEVICE
        assert ls(T(*([8] * 8)), 8) == bl.BL_ERR_DEVICE


def test_lut_rejects_and_limits(bl):
    lib = bl.library()
    f = lambda **kw: lib.bitlinear_forward_lut(kw.get("xq", P), P, P, kw.get("layout", 1), P,
                                               kw.get("M", 1), kw.get("N", 16), kw.get("K", 64),
                                               kw.get("y", P), 0, None, None)
    assert f(xq=None) == bl.BL_ERR_INVALID_ARG
    assert f(y=P + 4) == bl.BL_ERR_INVALID_ARG
    assert f(K=0) == bl.BL_ERR_INVALID_ARG
    assert f(layout=5) == bl.BL_ERR_INVALID_ARG
    assert f(layout=0) == bl.BL_ERR_UNSUPPORTED
    assert f(layout=2) == bl.BL_ERR_UNSUPPORTED
    assert f(M=2) == bl.BL_ERR_UNSUPPORTED
    assert f(M=0) == bl.BL_OK and f(N=0) == bl.BL_OK


def test_forward_plan_names_the_kernels(bl):
    """The dry run of the dispatch names the launches, without a GPU, for
    shapes whose launch shape does not depend on the compute-unit count."""
    import torch
    plan = bl.bitlinear_forward_plan(2048, 11008, 4096, "2bit", torch.bfloat16)
    assert len(plan) == 1 and plan[0].startswith("gemm_dma_pair_kernel<0, 96, false, unsigned short>")
    assert "(256 tiles 256x256 + 242 tiles 96x256)" in plan[0]
    plan = bl.bitlinear_forward_plan(4096, 4096, 4096, "2bit", torch.bfloat16)
    assert plan == ["gemm_dma_kernel<0, 256, false, unsigned short> grid=256x1 block=512 lds=132096"]
    plan = bl.bitlinear_forward_plan(4096, 4096, 4096, "base3", torch.bfloat16)
    assert plan == ["gemm_kernel<1, 256, 256, 1, 8, 2, 1, 0, unsigned short> grid=256x1 "
                    "block=512 lds=" + plan[0].split("lds=")[1]]
    plan = bl.bitlinear_forward_plan(1, 4096, 4096, "2bit", torch.float32, fused=True)
    assert plan[0].startswith("linear_decode_kernel<0, 8, 2, 1, false, 1, unsigned short, float> "
                              "grid=256x1 block=512")
    plan = bl.bitlinear_forward_plan(16, 12288, 4096, "2bit", torch.bfloat16)
    assert plan[0].startswith("skinny_kernel<0, 16, 1, 3, 16, false, unsigned short> grid=256x1")
    plan = bl.bitlinear_forward_plan(16, 4096, 11008, "2bit", torch.bfloat16)
    assert plan[0].startswith("skinny_kernel<0, 16, 1, 1, 16, true, unsigned short> grid=256x1")
    assert bl.bitlinear_forward_plan(0, 5, 5) == []
    with pytest.raises(bl.BitLinearError):
        bl.bitlinear_forward_plan(5, 4096, 4096, fused=True)


@pytest.mark.parametrize("layout", ["2bit", "1bit", "base3"])
@pytest.mark.parametrize("M,N", [(70000, 200), (70000, 256), (65600, 100), (300 * 256, 256)])
def test_forward_plan_never_launches_an_empty_grid(bl, layout, M, N):
    """Many row tiles over one column of tiles: no launch has zero blocks and
    the launches cover every column (an M past 256 tiles of 256 rows that is
    not a whole number of rounds once left a 256 x 256 launch over 0 columns)."""
    plan = bl.bitlinear_forward_plan(M, N, 256, layout)
    assert plan
    for line in plan:
        gx = int(line.split("grid=")[1].split("x")[0])
        assert gx > 0, line


def test_noalloc_pack_rejects(bl):
    """The allocation-free pack validates like the workspace pack, before any
    device call."""
    lib = bl.library()
    args = dict(W=P, w_dtype=1, N=8, K=64, scheme=0, layout=0, eps=1e-5, packed=P, gamma=P)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.bitlinear_pack_weights_noalloc(
            a["W"], a["w_dtype"], a["N"], a["K"], a["scheme"], a["layout"], a["eps"], a["packed"],
            a["gamma"], None)

    assert call(W=None) == bl.BL_ERR_INVALID_ARG
    assert call(packed=P + 8) == bl.BL_ERR_INVALID_ARG
    assert call(N=0) == bl.BL_ERR_INVALID_ARG
    assert call(K=16909321) == bl.BL_ERR_INVALID_ARG
    assert call(layout=2, scheme=0) == bl.BL_ERR_INVALID_ARG  # 1-bit holds binary codes only
    assert call(eps=float("nan")) == bl.BL_ERR_INVALID_ARG
    assert call(w_dtype=5) == bl.BL_ERR_INVALID_ARG
    assert bl.bitlinear_pack_noalloc_max_scratch_bytes() == 16384
    # the largest shape still fits: the mean never uses more than 1024 partials
    assert bl.bitlinear_pack_workspace_bytes(1 << 20, 1 << 20) <= 16384
    import torch
    if not torch.cuda.is_available():
        assert call() == bl.BL_ERR_DEVICE  # valid arguments, no gfx950 device
