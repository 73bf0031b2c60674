"""Parity at every launch configuration the benchmark times.

Each case runs one of bench.py's timed calls with the same seeded inputs,
shapes, layouts and output types, asserts (through the dispatch's dry run,
bitlinear_forward_plan) which kernel instantiation and grid serve it, and
compares the result with the oracle:

- decode, one token against 4096 x 4096: the fused step (2-bit, base-3, 1-bit
  layout) and the two-launch step (quantise, then the decode product);
- one token against a 32768 x 4096 matrix (2-bit and 1-bit layouts);
- prefill, 2048 x 11008 x 4096, bf16 out, all three layouts;
- one transformer block's six projections at one decode token (fused launches),
  decode batch 16 and prefill 512:
  Q|K|V stacked as three segments with their own weight scales, O, up, down
  ([b158] §5.4 replaces exactly these linear layers with BitLinear);
- the training shape's INT8 forward, 4096 x 4096 x 4096.

Outputs sit between guard bytes. Where the oracle would take minutes (M >= 512)
accumulators and outputs are compared on sampled token rows, every column;
codes, activation codes and scales are always compared in full.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import (SCALE_RTOL, check_codes, check_rel, check_y_bf16, check_y_f32, guarded,
                         to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def dev(a: np.ndarray, bf16: bool) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def kernel_of(plan_line: str) -> str:
    return plan_line.split(" grid=")[0]


def pack_segments(bl, ws, layout, scheme):
    """Pack each weight matrix into its row range of one stacked buffer, its
    scale into consecutive floats. Returns (packed, gammas, oracle codes, flags,
    oracle scales)."""
    K = ws[0].K
    rb = bl.bitlinear_packed_row_bytes(K, layout)
    N = sum(w.N for w in ws)
    packed, gpk = guarded((N, rb), torch.uint8)
    gammas, gg = guarded((max(4, len(ws)),), torch.float32)
    row = 0
    codes, flags, g_ref = [], [], []
    for s, w in enumerate(ws):
        bl.bitlinear_pack_weights(dev(w.w_store, w.dtype == "bf16"), layout, scheme,
                                  packed=packed[row:row + w.N], gamma=gammas[s:s + 1])
        if scheme == "ternary":
            c, f, g = oracle.ternary_codes(w.w)
        else:
            c, f, _a, g = oracle.binary_codes(w.w)
        codes.append(c)
        flags.append(f)
        g_ref.append(g)
        row += w.N
    torch.cuda.synchronize()
    gpk.check("packed", all_written=False)  # any byte value is a valid code byte
    gg.check("gammas", all_written=False)   # only the first len(ws) floats are written
    return packed, gammas, codes, flags, np.array(g_ref, np.float32)


def check_case(bl, name, ws, xp, layout, scheme, out_dtype, fused, expect_kernel,
               expect_grid=None, rows=None):
    """Run one benchmarked call (fused step, or quantise + product; stacked when
    len(ws) > 1) and compare it with the oracle."""
    M, K = xp.M, xp.K
    N = sum(w.N for w in ws)
    plan = bl.bitlinear_forward_plan(M, N, K, layout, out_dtype, fused=fused)
    print(f"[case] {name}: M={M} N={N} K={K} {layout} -> {plan}", flush=True)
    assert len(plan) == 1 and kernel_of(plan[0]) == expect_kernel, plan
    if expect_grid is not None:
        assert f" grid={expect_grid} " in plan[0], plan
    packed, gammas, codes, wflags, g_ref = pack_segments(bl, ws, layout, scheme)
    g_gpu = to_np(gammas)[:len(ws)]
    check_rel(g_gpu, g_ref, SCALE_RTOL, "weight scales")
    got_codes, bad = oracle.unpack(to_np(packed), K, layout)
    assert bad == 0
    all_codes = np.concatenate(codes, axis=0)
    check_codes(got_codes, all_codes, np.concatenate(wflags, axis=0), "codes")
    code_bad_cols = (got_codes != all_codes).any(axis=1)

    x = dev(xp.x_store, xp.dtype == "bf16")
    y, gy = guarded((M, N), out_dtype)
    acc, ga = guarded((M, N), torch.int32)
    segs = tuple(w.N for w in ws)
    xq_ref, s_ref, xflags = oracle.quant_acts(xp.x)
    if fused:
        if len(ws) > 1:
            bl.bitlinear_linear_segmented(x, packed, gammas, segs, layout, y=y, acc=acc)
        else:
            bl.bitlinear_linear(x, packed, gammas, N, layout, y=y, acc=acc)
        xq_bad_rows = np.zeros(M, bool)  # same fp32 steps as the oracle's
    else:
        xq, gq = guarded((M, K), torch.int8)
        sc, gs = guarded((M,), torch.float32)
        bl.bitlinear_quant_acts(x, xq=xq, scale=sc)
        if len(ws) > 1:
            bl.bitlinear_forward_segmented(xq, sc, packed, gammas, segs, K, layout, y=y, acc=acc)
        else:
            bl.bitlinear_forward(xq, sc, packed, gammas, N, K, layout, y=y, acc=acc)
        torch.cuda.synchronize()
        gq.check("xq", all_written=False)  # an activation code may equal the pattern byte
        gs.check("scale")
        check_codes(to_np(xq), xq_ref, xflags, "xq")
        assert np.array_equal(to_np(sc), s_ref)
        xq_bad_rows = (to_np(xq) != xq_ref).any(axis=1)
    torch.cuda.synchronize()
    gy.check("y")
    ga.check("acc")

    if rows is None:
        rows = np.arange(M)
    acc_ref = oracle.int_product(xq_ref[rows], all_codes)
    keep_r = ~xq_bad_rows[rows]
    keep_c = ~code_bad_cols
    got_acc = to_np(acc)[rows]
    assert np.array_equal(got_acc[keep_r][:, keep_c], acc_ref[keep_r][:, keep_c]), \
        "INT32 accumulators differ"
    parts, col = [], 0
    for w, g in zip(ws, g_ref):
        parts.append(oracle.epilogue(acc_ref[:, col:col + w.N], g, s_ref[rows]))
        col += w.N
    y64 = np.concatenate(parts, axis=1)
    if out_dtype == torch.float32:
        got_y = to_np(y)[rows]
        check_y_f32(got_y[keep_r][:, keep_c], y64[keep_r][:, keep_c])
    else:
        got_y = to_np(y.view(torch.int16)).view(np.uint16)[rows]
        check_y_bf16(got_y[keep_r][:, keep_c], y64[keep_r][:, keep_c])


def sample_rows(M, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n, replace=False)]))


SCHEME = {"2bit": "ternary", "base3": "ternary", "1bit": "binary"}


# ---------------------------------------------------------------- decode, C2
@pytest.mark.parametrize("layout", ["2bit", "base3", "1bit"])
def test_bench_decode_fused_step(bl, layout):
    """The headline step: one token, 4096 x 4096, fused quantise + product."""
    p = synth.workload("decode")
    L = {"2bit": 0, "base3": 1, "1bit": 2}[layout]
    check_case(bl, f"decode fused {layout}", [p], p, layout, SCHEME[layout], torch.float32, True,
               f"linear_decode_kernel<{L}, 8, 2, 1, false, 1, unsigned short, float>", "256x1")


@pytest.mark.parametrize("layout", ["2bit", "base3", "1bit"])
def test_bench_decode_two_launch_step(bl, layout):
    """The same step as two launches: the quantiser, then the decode product."""
    p = synth.workload("decode")
    L = {"2bit": 0, "base3": 1, "1bit": 2}[layout]
    check_case(bl, f"decode two-launch {layout}", [p], p, layout, SCHEME[layout], torch.float32,
               False, f"skinny_kernel<{L}, 8, 2, 1, 4, false, float>", "256x1")


@pytest.mark.parametrize("layout", ["2bit", "1bit"])
def test_bench_weight_stream_32768(bl, layout):
    """One token against 32768 x 4096 (the benchmark's 32 MiB stream)."""
    p = synth.make_problem(M=1, N=32768, K=4096, seed=9, dtype="bf16", outlier_frac=0.01)
    L = {"2bit": 0, "1bit": 2}[layout]
    check_case(bl, f"stream 32768x4096 {layout}", [p], p, layout, SCHEME[layout], torch.float32,
               True, f"linear_decode_kernel<{L}, 4, 4, 1, false, 2, unsigned short, float>",
               "1024x1")


# --------------------------------------------------------------- prefill, C3
@pytest.mark.parametrize("layout,kernel", [
    ("2bit", "gemm_dma_pair_kernel<0, 96, false, unsigned short> (256 tiles 256x256 + 242 tiles 96x256)"),
    ("base3", "gemm_pair_kernel<1, 0, unsigned short, 96> (256 tiles 256x256 + 242 tiles 96x256)"),
    ("1bit", "gemm_dma_pair_kernel<2, 96, false, unsigned short> (256 tiles 256x256 + 242 tiles 96x256)"),
])
def test_bench_prefill(bl, layout, kernel):
    p = synth.workload("prefill")
    check_case(bl, f"prefill {layout}", [p], p, layout, SCHEME[layout], torch.bfloat16, False,
               kernel, rows=sample_rows(p.M, 14, 3))


# ------------------------------------------------------ transformer block, C4
def block_inputs(M, K):
    # the benchmark's block inputs: bf16 N(0, 1), seed 77 + K
    return synth.make_problem(M=M, N=1, K=K, seed=77 + K, dtype="bf16")


BLOCK_1 = {  # one token, fused quantise + multiply per launch
    "qkv": "linear_decode_kernel<0, 4, 4, 1, false, 1, unsigned short, unsigned short>",
    "o": "linear_decode_kernel<0, 8, 2, 1, false, 1, unsigned short, unsigned short>",
    "up": "linear_decode_kernel<0, 4, 4, 1, false, 1, unsigned short, unsigned short>",
    "down": "linear_decode_kernel<0, 16, 1, 1, false, 1, unsigned short, unsigned short>",
}
BLOCK_16 = {
    "qkv": "skinny_kernel<0, 16, 1, 3, 16, false, unsigned short>",
    "o": "skinny_kernel<0, 16, 1, 1, 16, false, unsigned short>",
    "up": "skinny_kernel<0, 16, 1, 3, 16, false, unsigned short>",
    "down": "skinny_kernel<0, 16, 1, 1, 16, true, unsigned short>",
}
BLOCK_512 = {
    # (the dry run takes no segments: the stacked Q|K|V launch runs the same
    # tiles in the instantiation that picks each row's weight scale, "true")
    "qkv": "gemm_dma_kernel<0, 128, false, unsigned short>",
    "o": "gemm_kernel<0, 32, 128, 1, 4, 2, 1, 0, unsigned short>",
    "up": "gemm_dma_kernel<0, 128, false, unsigned short>",
    "down": "gemm_kernel<0, 64, 128, 1, 4, 2, 2, 0, unsigned short>",
}


@pytest.mark.parametrize("M", [1, 16, 512])
@pytest.mark.parametrize("part", ["qkv", "o", "up", "down"])
def test_bench_block(bl, M, part):
    """The block's launches as the benchmark makes them: Q|K|V as one stacked
    matrix of three segments with three weight scales, then O, up and down;
    2-bit codes, bf16 out. One token runs each as one fused launch (the launch
    shape counts tiles against the compute units of an MI355X)."""
    if M == 1 and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the one-token launch shape counts tiles against 256 compute units")
    idx = {"qkv": [0, 1, 2], "o": [3], "up": [4], "down": [5]}[part]
    ws = [synth.block_layer(i, 1) for i in idx]
    xp = block_inputs(M, ws[0].K)
    kernel = {1: BLOCK_1, 16: BLOCK_16, 512: BLOCK_512}[M][part]
    rows = None if M <= 16 else sample_rows(M, 8, 100 + idx[0])
    check_case(bl, f"block M={M} {part}", ws, xp, "2bit", "ternary", torch.bfloat16, M == 1,
               kernel, rows=rows)


# ------------------------------------------------------------- training, C5
def test_bench_train_forward(bl):
    """The training step's INT8 forward at 4096 x 4096 x 4096 (one round of
    256 x 256 tiles)."""
    t = synth.workload("train")
    check_case(bl, "train forward 4096^3", [t], t, "2bit", "ternary", torch.bfloat16, False,
               "gemm_dma_kernel<0, 256, false, unsigned short>", "256x1",
               rows=sample_rows(t.M, 8, 5))
