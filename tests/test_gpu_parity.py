"""GPU parity: the HIP path (through the C ABI binding) against the CPU oracle
on the same seeded inputs. Bars are stated in parity_util."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import (check_codes, check_rel, check_y_bf16, check_y_f32, excluded_acc_mask,
                         to_np, SCALE_RTOL)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def y_bits(y: torch.Tensor) -> np.ndarray:
    return to_np(y.view(torch.int16)).view(np.uint16)


def banner(msg):
    print(f"[case] {msg}", flush=True)


# ----------------------------------------------------------------------------
PACK_CASES = [
    (256, 256, "f32"), (37, 1000, "bf16"), (5, 17, "f32"), (3, 1, "f32"), (64, 80, "f32"),
    (129, 4099, "bf16"), (1, 65, "bf16"),
]


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("scheme", ["ternary", "binary"])
@pytest.mark.parametrize("N,K,dtype", PACK_CASES)
def test_pack_parity(bl, layout, scheme, N, K, dtype):
    banner(f"pack {layout} {scheme} N={N} K={K} {dtype}")
    p = synth.make_problem(M=1, N=N, K=K, seed=100 + N + K, dtype=dtype)
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, dtype == "bf16"), layout, scheme)
    torch.cuda.synchronize()
    if scheme == "ternary":
        codes, flags, g_ref = oracle.ternary_codes(p.w)
    else:
        codes, flags, _alpha, g_ref = oracle.binary_codes(p.w)
    g = to_np(gamma)[0]
    check_rel([g], [g_ref], SCALE_RTOL, "gamma")
    got = to_np(packed)
    codes_gpu, bad = oracle.unpack(got, K, layout)
    assert bad == 0
    n_ex = check_codes(codes_gpu, codes, flags, "codes")
    assert n_ex == 0 or g != g_ref
    assert np.array_equal(oracle.pack(codes_gpu, layout), got), "layout/padding differs"


def test_pack_deterministic(bl):
    p = synth.make_problem(M=1, N=300, K=700, seed=7, dtype="bf16")
    W = dev(p.w_store, True)
    a, ga = bl.bitlinear_pack_weights(W, "2bit")
    b, gb = bl.bitlinear_pack_weights(W, "2bit")
    assert torch.equal(a, b) and torch.equal(ga, gb)


def test_pack_zero_matrix(bl):
    W = torch.zeros((16, 96), dtype=torch.float32, device="cuda")
    packed, gamma = bl.bitlinear_pack_weights(W, "2bit")
    assert to_np(gamma)[0] == 0.0
    codes, bad = oracle.unpack(to_np(packed), 96, "2bit")
    assert bad == 0 and not codes.any()


# ----------------------------------------------------------------------------
QUANT_CASES = [(8, 256, "f32", 0.0), (1, 4096, "bf16", 0.01), (3, 17, "f32", 0.0),
               (5, 1000, "bf16", 0.0), (257, 64, "bf16", 0.0), (2, 20000, "f32", 0.0),
               (4, 11008, "bf16", 0.01)]


@pytest.mark.parametrize("M,K,dtype,outl", QUANT_CASES)
def test_quant_acts_parity(bl, M, K, dtype, outl):
    banner(f"quant M={M} K={K} {dtype}")
    p = synth.make_problem(M=M, N=1, K=K, seed=200 + M + K, dtype=dtype, outlier_frac=outl)
    x_store = p.x_store.copy()
    x_ref = p.x.copy()
    if M >= 3:  # one all-zero token
        x_store[1] = 0
        x_ref[1] = 0.0
    xq, scale = bl.bitlinear_quant_acts(dev(x_store, dtype == "bf16"))
    torch.cuda.synchronize()
    xq_ref, s_ref, flags = oracle.quant_acts(x_ref)
    check_rel(to_np(scale), s_ref, SCALE_RTOL, "scale")
    assert np.array_equal(to_np(scale), s_ref)  # a max is exact
    n_ex = check_codes(to_np(xq), xq_ref, flags, "xq")
    assert n_ex == 0, "same fp32 steps on both sides: no boundary mismatch expected"


@pytest.mark.parametrize("fused", [False, True])
def test_quant_acts_half_integer_boundaries(bl, fused):
    """Activations placed on and one ulp around x = s (k + 1/2) / 127 for every
    k, where the code is decided by the last bit of the fp32 quotient and the
    round-half-to-even rule: every code must equal the oracle's (IEEE division
    in the pages' order), boundary elements included."""
    banner(f"quant half-integer boundaries fused={fused}")
    rng = np.random.default_rng(4242)
    rows = []
    for s in (np.float32(127.0), np.float32(1.0), np.float32(3.7), np.float32(20.0),
              np.float32(0.0123), np.float32(1e-3)):
        k = np.arange(-127, 127, dtype=np.float64)
        base = (s.astype(np.float64) * (k + 0.5) / 127.0).astype(np.float32)
        vals = np.concatenate([base, np.nextafter(base, np.float32(np.inf)),
                               np.nextafter(base, np.float32(-np.inf))])
        vals = vals[np.abs(vals) <= s]
        row = np.zeros(1024, np.float32)
        row[:vals.size] = rng.permutation(vals)
        row[vals.size] = s  # the row maximum fixes the scale
        rows.append(row)
    x = np.stack(rows).astype(np.float32)
    xq_ref, s_ref, flags = oracle.quant_acts(x)
    assert flags.any()  # the case does exercise rounding boundaries
    if not fused:
        xq, scale = bl.bitlinear_quant_acts(dev(x))
        torch.cuda.synchronize()
        assert np.array_equal(to_np(scale), s_ref)
        assert np.array_equal(to_np(xq), xq_ref), "codes differ at a rounding boundary"
    else:
        # the fused decode step quantises inside the product: compare through
        # the accumulators against single-code weight rows (acc = one code)
        K = x.shape[1]
        for t in range(0, x.shape[0], 4):
            xs = np.ascontiguousarray(x[t:t + 4])
            M = xs.shape[0]
            codes = np.zeros((K, K), np.int8)
            np.fill_diagonal(codes, 1)
            packed = oracle.pack(codes, "2bit")
            g = torch.tensor([1.0, 0, 0, 0], dtype=torch.float32, device="cuda")
            y, acc = bl.bitlinear_linear(dev(xs), dev(packed), g, K, "2bit", acc=True)
            torch.cuda.synchronize()
            assert np.array_equal(to_np(acc), xq_ref[t:t + M].astype(np.int32)), \
                "fused codes differ at a rounding boundary"


# ----------------------------------------------------------------------------
FWD_CASES = [
    (1, 256, 256), (1, 31, 100), (2, 300, 1000), (3, 64, 64), (5, 16, 1), (8, 256, 256),
    (16, 100, 4096), (16, 33, 17), (17, 256, 256), (64, 130, 1000), (130, 300, 260),
    (257, 257, 320), (33, 1, 160), (128, 128, 4096), (300, 512, 129),
    # medium batches: the weight-streaming kernel in 16-token chunks (partial
    # last chunk, six chunks, eight chunks over long rows) or, past the
    # measured crossover, the GEMM (many rows; base-3 switches earlier)
    (17, 4096, 512), (96, 512, 4096), (40, 20000, 64), (33, 17000, 100), (31, 40000, 32),
    (64, 20000, 64), (120, 1000, 9000),
    # enough 256 x 256 tiles for a full round plus leftover columns (a second
    # launch, or one paired launch when the leftover fills a round of 128 x 256)
    (4096, 4357, 64), (2048, 8200, 48), (2000, 11000, 48), (2048, 11008, 40),
    (2048, 11192, 48), (8192, 2048, 128),
    # many rows at M <= 4 (the four-wave weight-streaming launch shape)
    (2, 16400, 96), (1, 16384, 33),
    # long rows (64 or more k-tiles) over few tiles: two wave groups split each
    # tile's k-tiles in the GEMM (odd k-tile counts, ragged K, edge tiles; an
    # odd number of base-3 units at K = 8192). Base-3 takes the chunked
    # weight-streaming product for the narrower of these and the GEMM from
    # chunks x rows > 16384 on.
    (130, 300, 9001), (200, 520, 8192), (130, 256, 10400), (150, 700, 12001), (97, 64, 16384),
    (130, 1900, 8192), (130, 2000, 10400),
    # 33 k-tiles over few tiles (2-bit at K = 4224, base-3 at K = 5280): two
    # wave groups split them (2-bit 32 x 128 tiles, base-3 64 x 128)
    (256, 256, 4224), (256, 1100, 5280),
    # an odd number of k-tiles on whole tiles under one wave group: the last
    # step runs alone, unguarded (2-bit 32 x 128 tiles, 3 k-tiles; base-3 takes
    # its guarded path at K = 384)
    (300, 300, 384),
    # rows of K % 16 != 0 bytes but 4-byte aligned (dword loads), beside the
    # byte-wise odd K above
    (300, 700, 2052), (257, 1000, 4100),
    # base-3 with 160 to 256 tiles of 128 x 128: two groups split each tile's
    # k-tiles (whole and ragged rows; 2-bit takes 32 x 128 tiles here)
    (1280, 2048, 160), (1200, 2000, 333),
    # long rows with at most half a round of 128 x 64 tiles: 2-bit takes
    # 64 x 64 tiles with split k-tiles (edge tiles in both directions; the
    # dispatch counts 128 x 64 and 64 x 64 tiles and launches 64 x 128 and
    # 32 x 128 tiles of the same area)
    (250, 1000, 8200),
    # at most one round of 64 x 64 tiles (2-bit) or half a round of 128 x 64
    # tiles (base-3) over 32 or more k-tiles: split k-tiles at K = 4096, on
    # ragged rows and at K = 6000
    (200, 1000, 4096), (192, 900, 5000), (200, 1000, 6000),
    # ragged rows split from 16 k-tiles on
    (200, 2000, 3000),
    # one chunk of 5-16 tokens on sixteen waves of one load per lane: three
    # row groups over rows longer than a round (2-bit) or one round (base-3),
    # one row group over long ragged rows
    (7, 9000, 4100), (9, 700, 9001),
]


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("M,N,K", FWD_CASES)
def test_forward_stage_parity(bl, layout, M, N, K):
    """Both sides get the same codes, activations, scales and gamma: the INT32
    accumulators must be bit-exact and y within the output tolerance."""
    banner(f"forward {layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    scale = rng.uniform(0.5, 30.0, size=M).astype(np.float32)
    gamma = np.float32(0.0161)
    packed = oracle.pack(codes, layout)
    g = torch.tensor([gamma, 0, 0, 0], dtype=torch.float32, device="cuda")
    acc_ref = oracle.int_product(xq, codes)
    y64 = oracle.epilogue(acc_ref, gamma, scale)
    for ydt in (torch.float32, torch.bfloat16):
        y, acc = bl.bitlinear_forward(dev(xq), dev(scale), dev(packed), g, N, K, layout, ydt,
                                      acc=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(acc), acc_ref), "INT32 accumulators differ"
        if ydt == torch.float32:
            check_y_f32(to_np(y), y64)
        else:
            check_y_bf16(y_bits(y), y64)


@pytest.mark.parametrize("layout", ["2bit", "base3", "1bit"])
def test_forward_long_rows_sampled(bl, layout):
    """1024 tokens x 2560 rows x K = 8200 (ragged): 128 x 128 tiles whose
    k-tiles two wave groups split. Accumulators and bf16 outputs on 24 token
    rows spread over every 128-token tile (first and last rows included)."""
    M, N, K = 1024, 2560, 8200
    banner(f"forward long rows {layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(8200)
    if layout == "1bit":
        codes = np.where(rng.random((N, K)) < 0.5, -1, 1).astype(np.int8)
    else:
        codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    scale = rng.uniform(0.5, 30.0, size=M).astype(np.float32)
    gamma = np.float32(0.0123)
    g = torch.tensor([gamma, 0, 0, 0], dtype=torch.float32, device="cuda")
    y, acc = bl.bitlinear_forward(dev(xq), dev(scale), dev(oracle.pack(codes, layout)), g, N, K,
                                  layout, torch.bfloat16, acc=True)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, M - 1], 128 * np.arange(8) + rng.integers(0, 128, size=8),
                           rng.choice(M, 14, replace=False)])
    acc_ref = oracle.int_product(xq[rows], codes)
    assert np.array_equal(to_np(acc)[rows], acc_ref), "INT32 accumulators differ"
    check_y_bf16(y_bits(y)[rows], oracle.epilogue(acc_ref, gamma, scale[rows]))


@pytest.mark.parametrize("layout,M,N,K,kernel", [
    # one round of 128 x 128 tiles, one wave group, whole k-tiles
    ("2bit", 1000, 4096, 4096, "gemm_kernel<0, 128, 128, 1, 4, 2, 1, 0, unsigned short>"),
    ("1bit", 1000, 4096, 4096, "gemm_kernel<2, 128, 128, 1, 4, 2, 1, 0, unsigned short>"),
    # many row tiles over one column of tiles, not a whole number of rounds
    ("2bit", 70000, 200, 256, "gemm_kernel<0, 128, 128, 1, 4, 2, 1, 0, unsigned short>"),
    ("1bit", 70000, 200, 256, "gemm_kernel<2, 128, 128, 1, 4, 2, 1, 0, unsigned short>"),
    ("base3", 70000, 200, 256, "gemm_kernel<1, 128, 256, 1, 8, 2, 1, 0, unsigned short>"),
    # whole rounds of 256 x 256 tiles in the base-3 layout
    ("base3", 4096, 4096, 4096, "gemm_kernel<1, 256, 256, 1, 8, 2, 1, 0, unsigned short>"),
    # one launch of 256 x 256 tiles plus the leftover columns: 96-row leftover
    # tiles where they make one round (ragged last row tile), else 128-row ones
    ("2bit", 2000, 11000, 256,
     "gemm_pair_kernel<0, 0, unsigned short, 96> (256 tiles 256x256 + 231 tiles 96x256)"),
    ("base3", 2000, 11000, 200,
     "gemm_pair_kernel<1, 2, unsigned short, 96> (256 tiles 256x256 + 231 tiles 96x256)"),
    ("1bit", 2000, 11000, 256,
     "gemm_pair_kernel<2, 0, unsigned short, 96> (256 tiles 256x256 + 231 tiles 96x256)"),
    ("2bit", 2048, 11192, 256,
     "gemm_pair_kernel<0, 0, unsigned short, 128> (256 tiles 256x256 + 192 tiles 128x256)"),
    # whole 256 x 256 tiles, whole k-tiles, bf16 out: activations by direct-to-LDS
    # loads through three stages (k-tile counts 1, 3 = one unrolled pass, 5 = a
    # pass and both tail steps, 32; two rounds of tiles)
    ("2bit", 8192, 2048, 128, "gemm_dma_kernel<0, 256, false, unsigned short>"),
    ("1bit", 4096, 4096, 384, "gemm_dma_kernel<2, 256, false, unsigned short>"),
    ("1bit", 8192, 2048, 640, "gemm_dma_kernel<2, 256, false, unsigned short>"),
    ("2bit", 4096, 4096, 4096, "gemm_dma_kernel<0, 256, false, unsigned short>"),
    ("2bit", 8192, 4096, 512, "gemm_dma_kernel<0, 256, false, unsigned short>"),
    # the same tiles with ragged token rows: the one-launch pair with 96-row
    # leftover tiles (2-bit) and 128-row ones (1-bit), and 128 x 256 tiles
    ("2bit", 2000, 11008, 256,
     "gemm_dma_pair_kernel<0, 96, false, unsigned short> (256 tiles 256x256 + 231 tiles 96x256)"),
    ("1bit", 2040, 11264, 128,
     "gemm_dma_pair_kernel<2, 128, false, unsigned short> (256 tiles 256x256 + 192 tiles 128x256)"),
    ("2bit", 500, 12288, 256, "gemm_dma_kernel<0, 128, false, unsigned short>"),
])
def test_forward_large_sampled(bl, layout, M, N, K, kernel):
    """Dispatch cases too large for a full oracle product: the configuration is
    asserted through the dispatch's dry run, accumulators and bf16 outputs are
    compared on sampled token rows (first and last included), every column."""
    banner(f"forward sampled {layout} M={M} N={N} K={K}")
    plan = bl.bitlinear_forward_plan(M, N, K, layout, torch.bfloat16)
    assert len(plan) == 1 and plan[0].split(" grid=")[0] == kernel, plan
    rng = np.random.default_rng(M + N + K)
    if layout == "1bit":
        codes = np.where(rng.random((N, K)) < 0.5, -1, 1).astype(np.int8)
    else:
        codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    scale = rng.uniform(0.5, 30.0, size=M).astype(np.float32)
    gamma = np.float32(0.0137)
    g = torch.tensor([gamma, 0, 0, 0], dtype=torch.float32, device="cuda")
    y, acc = bl.bitlinear_forward(dev(xq), dev(scale), dev(oracle.pack(codes, layout)), g, N, K,
                                  layout, torch.bfloat16, acc=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    acc_ref = oracle.int_product(xq[rows], codes)
    assert np.array_equal(to_np(acc)[rows], acc_ref), "INT32 accumulators differ"
    check_y_bf16(y_bits(y)[rows], oracle.epilogue(acc_ref, gamma, scale[rows]))


# ----------------------------------------------------------------------------
def run_gpu_pipeline(bl, p, layout, scheme="ternary", out_dtype=torch.float32):
    bf = p.dtype == "bf16"
    W = dev(p.w_store, bf)
    x = dev(p.x_store, bf)
    packed, gamma = bl.bitlinear_pack_weights(W, layout, scheme)
    xq, scale = bl.bitlinear_quant_acts(x)
    y, acc = bl.bitlinear_forward(xq, scale, packed, gamma, p.N, p.K, layout, out_dtype,
                                  acc=True)
    torch.cuda.synchronize()
    return dict(packed=to_np(packed), gamma=to_np(gamma)[0], xq=to_np(xq), scale=to_np(scale),
                acc=to_np(acc), y=y)


def check_end_to_end(got, ref, p, layout, out_dtype):
    check_rel([got["gamma"]], [ref["gamma"]], SCALE_RTOL, "gamma")
    codes_gpu, bad = oracle.unpack(got["packed"], p.K, layout)
    assert bad == 0
    code_bad = codes_gpu != ref["codes"]
    check_codes(codes_gpu, ref["codes"], ref["wflags"], "codes")
    xq_bad = got["xq"] != ref["xq"]
    check_codes(got["xq"], ref["xq"], ref["xflags"], "xq")
    assert np.array_equal(got["scale"], ref["scale"])
    ex = excluded_acc_mask(xq_bad, code_bad)
    assert np.array_equal(got["acc"][~ex], ref["acc"][~ex])
    keep = ~ex
    y = got["y"]
    if out_dtype == torch.float32:
        check_y_f32(to_np(y)[keep], ref["y64"][keep])
    else:
        check_y_bf16(y_bits(y)[keep], ref["y64"][keep])
    return int(ex.sum())


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("scheme", ["ternary", "binary"])
def test_end_to_end_tiny(bl, layout, scheme):
    """M=8, K=256, N=256, fp32 inputs and output (the oracle's small workload)."""
    banner(f"e2e tiny {layout} {scheme}")
    p = synth.workload("tiny")
    got = run_gpu_pipeline(bl, p, layout, scheme)
    ref = oracle.forward(p.w, p.x, layout, scheme)
    assert check_end_to_end(got, ref, p, layout, torch.float32) == 0


@pytest.mark.parametrize("layout", ["2bit", "base3"])
def test_end_to_end_decode_full(bl, layout):
    """Decode GEMV at full size: M=1, 4096 x 4096, bf16 inputs with outliers."""
    banner(f"e2e decode {layout}")
    p = synth.workload("decode")
    got = run_gpu_pipeline(bl, p, layout)
    ref = oracle.forward(p.w, p.x, layout)
    assert check_end_to_end(got, ref, p, layout, torch.float32) == 0


@pytest.mark.parametrize("M", [16, 512])
def test_end_to_end_block_layer(bl, M):
    """The FFN down projection (K = 11008) at decode batch 16 and prefill 512."""
    banner(f"e2e block down M={M}")
    p = synth.block_layer(5, M)
    got = run_gpu_pipeline(bl, p, "2bit", out_dtype=torch.bfloat16)
    ref = oracle.forward(p.w, p.x, "2bit")
    check_end_to_end(got, ref, p, "2bit", torch.bfloat16)


@pytest.mark.parametrize("layout", ["2bit", "base3"])
def test_prefill_full_size_sampled(bl, layout):
    """Prefill at full size (M=2048, K=4096, N=11008, bf16 out): gamma, every
    code and every activation code are compared; accumulators and outputs on
    a sample of 24 token rows (all 11008 columns)."""
    banner(f"prefill full {layout}")
    p = synth.workload("prefill")
    got = run_gpu_pipeline(bl, p, layout, out_dtype=torch.bfloat16)
    codes, wflags, g_ref = oracle.ternary_codes(p.w)
    check_rel([got["gamma"]], [g_ref], SCALE_RTOL, "gamma")
    codes_gpu, bad = oracle.unpack(got["packed"], p.K, layout)
    assert bad == 0
    check_codes(codes_gpu, codes, wflags, "codes")
    xq_ref, s_ref, xflags = oracle.quant_acts(p.x)
    check_codes(got["xq"], xq_ref, xflags, "xq")
    assert np.array_equal(got["scale"], s_ref)
    rows = np.random.default_rng(0).choice(p.M, 24, replace=False)
    rows = np.concatenate([rows, [0, p.M - 1]])
    acc_ref = oracle.int_product(xq_ref[rows], codes)
    code_bad = codes_gpu != codes
    cols_ok = ~code_bad.any(axis=1)
    assert np.array_equal(got["acc"][rows][:, cols_ok], acc_ref[:, cols_ok])
    y64 = oracle.epilogue(acc_ref, g_ref, s_ref[rows])
    check_y_bf16(y_bits(got["y"])[rows][:, cols_ok], y64[:, cols_ok])


def test_zero_activation_row_gives_zero_output(bl):
    p = synth.make_problem(M=20, N=64, K=256, seed=3, dtype="f32")
    p.x_store[4] = 0.0
    got = run_gpu_pipeline(bl, p, "2bit")
    assert got["scale"][4] == np.float32(1e-6)
    assert not got["xq"][4].any() and not got["acc"][4].any()
    assert torch.all(got["y"][4] == 0)


# ----------------------------------------------------------------------------
# Fused decode step (quantise + multiply in one launch)
@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("M,N,K,dtype", [(1, 256, 256, "f32"), (2, 100, 1000, "bf16"),
                                         (3, 33, 17, "f32"), (4, 300, 4099, "bf16"),
                                         (1, 4096, 11008, "bf16"), (4, 64, 8192, "f32"),
                                         (1, 16400, 160, "bf16"), (3, 16384, 5000, "f32"),
                                         # one token, two 16-row groups per block; the
                                         # last block holds a single row
                                         (1, 16385, 4096, "f32"),
                                         # several tokens, four row groups per block
                                         (2, 32800, 256, "bf16"), (4, 32769, 100, "f32"),
                                         # several tokens, more 16-row tiles than the
                                         # capped grid (two blocks per compute unit):
                                         # blocks stream tiles; ragged last tile
                                         (2, 8200, 64, "bf16"), (3, 12000, 4096, "f32"),
                                         (4, 22016, 4096, "bf16"), (2, 9000, 5120, "bf16"),
                                         # one token: four waves of four loads over one-round
                                         # rows with more tiles than CUs; sixteen waves of one
                                         # load over longer rows with at most one tile per CU
                                         (1, 11008, 4096, "bf16"), (1, 6000, 1000, "f32"),
                                         (1, 300, 9001, "bf16"), (1, 4096, 8192, "f32")])
def test_fused_linear_parity(bl, layout, M, N, K, dtype):
    """Same activation codes as the stand-alone quantiser (bit-exact), hence
    the same INT32 accumulators as the oracle, and y within tolerance."""
    banner(f"fused {layout} M={M} N={N} K={K} {dtype}")
    p = synth.make_problem(M=M, N=N, K=K, seed=300 + M + N + K, dtype=dtype, outlier_frac=0.01)
    bf = dtype == "bf16"
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, bf), layout)
    y, acc = bl.bitlinear_linear(dev(p.x_store, bf), packed, gamma, N, layout, acc=True)
    torch.cuda.synchronize()
    ref = oracle.forward(p.w, p.x, layout)
    got = dict(packed=to_np(packed), gamma=to_np(gamma)[0], xq=ref["xq"], scale=ref["scale"],
               acc=to_np(acc), y=y)
    assert check_end_to_end(got, ref, p, layout, torch.float32) == 0


@pytest.mark.parametrize("N,K,shape", [(11008, 4096, "4, 4"), (6000, 1000, "4, 4"),
                                       (4096, 4096, "8, 2"), (4096, 8192, "16, 1"),
                                       (300, 9001, "16, 1")])
def test_fused_one_token_launch_shape(bl, N, K, shape):
    """One token: the launch shape (waves, loads per lane) the parity cases
    above reach, by the dispatch's dry run on this device."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the rule counts tiles against the compute units of an MI355X")
    plan = bl.bitlinear_forward_plan(1, N, K, "2bit", torch.float32, fused=True)
    assert plan[0].startswith(f"linear_decode_kernel<0, {shape}, 1, false, 1, "), plan


def test_fused_linear_decode_full(bl):
    """The decode workload (M=1, 4096 x 4096, bf16, outliers) through the fused path."""
    p = synth.workload("decode")
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, True), "2bit")
    y, acc = bl.bitlinear_linear(dev(p.x_store, True), packed, gamma, p.N, "2bit", acc=True)
    torch.cuda.synchronize()
    ref = oracle.forward(p.w, p.x, "2bit")
    assert np.array_equal(to_np(acc), ref["acc"])
    check_y_f32(to_np(y), ref["y64"])
