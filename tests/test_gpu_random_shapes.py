"""Seeded random shapes through every product path, against the oracle.

Each case draws a layout (2-bit, base-3, 1-bit with binary codes), input and
output dtypes, and M, N, K with ragged edges: M <= 4 runs the fused decode
step, 5 <= M <= 16 the decode product, larger M the tiled GEMM (both after
the stand-alone quantiser). Accumulators must match the oracle bit for bit
(outside elements on a rounding boundary, which are excluded and bounded as
in the other parity tests), outputs within the output tolerance."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import (SCALE_RTOL, check_codes, check_rel, check_y_bf16, check_y_f32,
                         excluded_acc_mask, guarded, to_np)

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


def draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = ["2bit", "base3", "1bit"][i % 3]
        band = i % 5  # fused, decode product, GEMM, GEMM with many rows, fused many rows
        M = [int(rng.integers(1, 5)), int(rng.integers(5, 17)), int(rng.integers(17, 130)),
             int(rng.integers(130, 400)), int(rng.integers(1, 5))][band]
        # many rows: the capped streaming grid and the two- and four-group blocks
        N = int(rng.integers(8000, 40000)) if band == 4 else int(rng.integers(1, 700))
        K = int(rng.integers(16, 700)) // 16 * 16 if band == 4 else int(rng.integers(1, 1300))
        cases.append((i, layout, M, N, K, ["f32", "bf16"][int(rng.integers(0, 2))],
                      [torch.float32, torch.bfloat16][int(rng.integers(0, 2))]))
    return cases


@pytest.mark.parametrize("case", draw_cases(60, 2024), ids=lambda c: f"{c[1]}-M{c[2]}-N{c[3]}-K{c[4]}")
def test_random_shape_parity(bl, case):
    i, layout, M, N, K, dtype, out_dtype = case
    print(f"[case] random {i}: {layout} M={M} N={N} K={K} {dtype} -> {out_dtype}", flush=True)
    scheme = "binary" if layout == "1bit" else "ternary"
    p = synth.make_problem(M=M, N=N, K=K, seed=5000 + i, dtype=dtype, outlier_frac=0.01)
    bf = dtype == "bf16"
    # every output sits between guard bytes (checked after the calls)
    packed, gpk = guarded((N, bl.bitlinear_packed_row_bytes(K, layout)), torch.uint8)
    gamma, gg = guarded((1,), torch.float32)
    bl.bitlinear_pack_weights(dev(p.w_store, bf), layout, scheme, packed=packed, gamma=gamma)
    x = dev(p.x_store, bf)
    ref = oracle.forward(p.w, p.x, layout, scheme)
    torch.cuda.synchronize()
    gpk.check("packed", all_written=False)  # any byte value is a valid code byte
    gg.check("gamma")
    codes_gpu, bad = oracle.unpack(to_np(packed), K, layout)
    assert bad == 0
    check_codes(codes_gpu, ref["codes"], ref["wflags"], "codes")
    y, gy_ = guarded((M, N), out_dtype)
    acc, ga = guarded((M, N), torch.int32)
    if M <= 4:
        bl.bitlinear_linear(x, packed, gamma, N, layout, y=y, acc=acc)
        xq_bad = np.zeros_like(ref["xq"], bool)  # same fp32 steps as the oracle
    else:
        xq, gq = guarded((M, K), torch.int8)
        scale, gs = guarded((M,), torch.float32)
        bl.bitlinear_quant_acts(x, xq=xq, scale=scale)
        bl.bitlinear_forward(xq, scale, packed, gamma, N, K, layout, y=y, acc=acc)
        torch.cuda.synchronize()
        gq.check("xq", all_written=False)  # codes may equal the pattern's byte
        gs.check("scale")
        check_codes(to_np(xq), ref["xq"], ref["xflags"], "xq")
        assert np.array_equal(to_np(scale), ref["scale"])
        xq_bad = to_np(xq) != ref["xq"]
    torch.cuda.synchronize()
    gy_.check("y")
    ga.check("acc")
    ex = excluded_acc_mask(xq_bad, codes_gpu != ref["codes"])
    assert np.array_equal(to_np(acc)[~ex], ref["acc"][~ex])
    if out_dtype == torch.float32:
        check_y_f32(to_np(y)[~ex], ref["y64"][~ex])
    else:
        check_y_bf16(to_np(y.view(torch.int16)).view(np.uint16)[~ex], ref["y64"][~ex])


def draw_branch_cases(n, seed):
    """Ragged shapes on the dispatch branches that pick a launch shape by size:
    one token over more 16-row tiles than compute units (four waves, four loads
    per lane) or over rows longer than a round (sixteen waves, one load), one
    chunk of 5-16 tokens (sixteen waves; one or three row groups), and
    prefill-like GEMMs with whole rounds of 256 x 256 tiles plus leftover
    columns (96- or 128-row leftover tiles)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = ["2bit", "base3", "1bit"][i % 3]
        kind = i % 4
        if kind == 0:
            M, N, K = 1, int(rng.integers(4097, 16384)), int(rng.integers(16, 4200))
        elif kind == 1:
            M, N, K = 1, int(rng.integers(1, 4097)), int(rng.integers(4097, 14000))
        elif kind == 2:
            N = int(rng.integers(1, 8192)) if i % 8 == 2 else int(rng.integers(8192, 12289))
            M, K = int(rng.integers(5, 17)), int(rng.integers(1, 9000))
        else:
            M, N, K = int(rng.integers(1800, 2300)), int(rng.integers(8300, 12300)), int(
                rng.integers(16, 80))
        cases.append((7000 + i, layout, M, N, K, ["f32", "bf16"][int(rng.integers(0, 2))],
                      [torch.float32, torch.bfloat16][int(rng.integers(0, 2))]))
    return cases


@pytest.mark.parametrize("case", draw_branch_cases(24, 31),
                         ids=lambda c: f"{c[1]}-M{c[2]}-N{c[3]}-K{c[4]}")
def test_random_launch_shape_parity(bl, case):
    test_random_shape_parity(bl, case)


def draw_lds_tile_cases(n, seed):
    """Ragged token rows on the GEMM tiles that take activations by
    direct-to-LDS loads: columns in whole 256-wide tiles, whole k-tiles (2-bit,
    and 1-bit without padding codes), bf16 out; enough tiles for 256 x 256
    rounds, the one-launch pair and 128 x 256 tiles."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = ["2bit", "1bit"][i % 2]
        M = int(rng.integers(380, 2300))
        N = 256 * int(rng.integers(24, 48))
        K = 128 * int(rng.integers(1, 4))
        cases.append((8000 + i, layout, M, N, K, ["f32", "bf16"][int(rng.integers(0, 2))],
                      torch.bfloat16))
    return cases


@pytest.mark.parametrize("case", draw_lds_tile_cases(12, 41),
                         ids=lambda c: f"{c[1]}-M{c[2]}-N{c[3]}-K{c[4]}")
def test_random_lds_tile_parity(bl, case):
    test_random_shape_parity(bl, case)


def draw_stacks(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        layout = ["2bit", "base3", "1bit"][i % 3]
        nseg = int(rng.integers(1, 9))
        big = i % 2 == 1
        segs = tuple(int(v) for v in rng.integers(1, 6000 if big else 300, size=nseg))
        M = int(rng.integers(1, 5)) if i % 4 < 2 else int(rng.integers(5, 200))
        K = int(rng.integers(1, 600))
        out.append((i, layout, M, segs, K))
    return out


@pytest.mark.parametrize("case", draw_stacks(24, 77),
                         ids=lambda c: f"{c[1]}-M{c[2]}-segs{len(c[3])}-K{c[4]}")
def test_random_stack_parity(bl, case):
    """Random stacks of 1..8 row segments, each with its own scale, through the
    segmented calls: the fused step for M <= 4 (from bf16 x), quantise + the
    segmented product otherwise. Every segment must equal the oracle on it."""
    i, layout, M, segs, K = case
    print(f"[case] random stack {i}: {layout} M={M} segs={segs} K={K}", flush=True)
    rng = np.random.default_rng(9000 + i)
    if layout == "1bit":  # binary codes only
        codes = [np.where(rng.random((n, K)) < 0.5, -1, 1).astype(np.int8) for n in segs]
    else:
        codes = [rng.integers(-1, 2, size=(n, K)).astype(np.int8) for n in segs]
    scales = np.zeros(max(4, (len(segs) + 3) // 4 * 4), np.float32)
    scales[:len(segs)] = rng.uniform(0.005, 0.05, size=len(segs))
    packed = dev(np.concatenate([oracle.pack(c, layout) for c in codes], axis=0), False)
    p = synth.make_problem(M=M, N=1, K=K, seed=9500 + i, dtype="bf16", outlier_frac=0.01)
    x = dev(p.x_store, True)
    y, gy_ = guarded((M, sum(segs)), torch.float32)
    acc, ga = guarded((M, sum(segs)), torch.int32)
    if M <= 4:
        bl.bitlinear_linear_segmented(x, packed, dev(scales, False), segs, layout, y=y, acc=acc)
    else:
        xq, scale = bl.bitlinear_quant_acts(x)
        bl.bitlinear_forward_segmented(xq, scale, packed, dev(scales, False), segs, K, layout,
                                       y=y, acc=acc)
    torch.cuda.synchronize()
    gy_.check("y")
    ga.check("acc")
    xq_ref, s_ref, _ = oracle.quant_acts(p.x)  # same fp32 steps on both sides
    acc_ref = oracle.int_product(xq_ref, np.concatenate(codes, axis=0))
    assert np.array_equal(to_np(acc), acc_ref)
    cols, parts = 0, []
    for c, g in zip(codes, scales):
        parts.append(oracle.epilogue(acc_ref[:, cols:cols + c.shape[0]], g, s_ref))
        cols += c.shape[0]
    check_y_f32(to_np(y), np.concatenate(parts, axis=1))


def draw_packs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        layout = ["2bit", "base3", "1bit"][i % 3]
        scheme = "binary" if layout == "1bit" else ["ternary", "binary"][int(rng.integers(0, 2))]
        out.append((i, layout, scheme, int(rng.integers(1, 400)), int(rng.integers(1, 3000)),
                    ["f32", "bf16"][int(rng.integers(0, 2))]))
    return out


@pytest.mark.parametrize("case", draw_packs(24, 31),
                         ids=lambda c: f"{c[1]}-{c[2]}-N{c[3]}-K{c[4]}-{c[5]}")
def test_random_pack_parity(bl, case):
    """Random shapes through the packer: the weight scale, every code (outside
    boundary flags) and every packed byte, padding included, against the
    oracle's layout."""
    i, layout, scheme, N, K, dtype = case
    print(f"[case] random pack {i}: {layout} {scheme} N={N} K={K} {dtype}", flush=True)
    p = synth.make_problem(M=1, N=N, K=K, seed=7000 + i, dtype=dtype)
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, dtype == "bf16"), layout, scheme)
    torch.cuda.synchronize()
    if scheme == "ternary":
        codes, flags, g_ref = oracle.ternary_codes(p.w)
    else:
        codes, flags, _alpha, g_ref = oracle.binary_codes(p.w)
    g = to_np(gamma)[0]
    check_rel([g], [g_ref], SCALE_RTOL, "weight scale")
    got = to_np(packed)
    codes_gpu, bad = oracle.unpack(got, K, layout)
    assert bad == 0
    assert check_codes(codes_gpu, codes, flags, "codes") == 0 or g != g_ref
    assert np.array_equal(oracle.pack(codes_gpu, layout), got)


def draw_bwd(n, seed):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 300)), int(rng.integers(1, 80)) * 8,
             int(rng.integers(1, 100)) * 8) for i in range(n)]


@pytest.mark.parametrize("case", draw_bwd(12, 5), ids=lambda c: f"M{c[1]}-N{c[2]}-K{c[3]}")
def test_random_backward_parity(bl, case):
    """Random shapes through both straight-through-estimator products, to the
    fp32 summation bound of the backward tests (n u sum|terms| + u |ref|)."""
    i, M, N, K = case
    print(f"[case] random backward {i}: M={M} N={N} K={K}", flush=True)
    u = 2.0 ** -24
    p = synth.make_problem(M=M, N=N, K=K, seed=8000 + i, dtype="bf16", grad_std=1e-3)
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, True), "2bit")
    gy = dev(p.grad_y_store, True)
    gx, ggx = guarded((M, K), torch.float32)
    gw, ggw = guarded((N, K), torch.float32)
    bl.bitlinear_backward_input(gy, packed, gamma, K, grad_x=gx)
    bl.bitlinear_backward_weight(gy, dev(p.x_store, True), grad_w=gw)
    torch.cuda.synchronize()
    ggx.check("grad_x")
    ggw.check("grad_w")
    codes, bad = oracle.unpack(to_np(packed), K, "2bit")
    assert bad == 0
    g = float(to_np(gamma)[0])
    ref = oracle.ste_grad_x(p.grad_y, codes, g)
    s = (np.abs(p.grad_y.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    err = np.abs(to_np(gx).astype(np.float64) - ref)
    assert np.all(err <= 1.01 * (N * u * s + u * np.abs(ref)) + 1e-30), "grad_x"
    ref = oracle.ste_grad_w(p.grad_y, p.x)
    s = np.abs(p.grad_y.astype(np.float64)).T @ np.abs(p.x.astype(np.float64))
    err = np.abs(to_np(gw).astype(np.float64) - ref)
    assert np.all(err <= 1.01 * (M * u * s + u * np.abs(ref)) + 1e-30), "grad_w"
