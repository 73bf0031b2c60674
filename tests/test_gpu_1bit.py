"""GPU parity of the 1-bit layout (BL_PACK_1BIT, binary codes of the 1-bit
BitLinear stored one bit per weight) against the oracle: packed bytes and
beta bit-exact, INT32 accumulators bit-exact, y within the output tolerance,
through every product path that reads the layout: the decode product (both
batch variants), the tiled GEMM (edge tiles, ragged K, and the prefill-size
one-launch pair of tile shapes), the fused decode step (one token, several
tokens streaming tiles, fp32 x, long rows) and stacked segments."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import (SCALE_RTOL, check_codes, check_rel, check_y_bf16, check_y_f32,
                         excluded_acc_mask, to_np)

pytestmark = pytest.mark.gpu
LAYOUT, SCHEME = "1bit", "binary"


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


def check_packed(bl, packed, gamma, p):
    """beta and the packed bytes against the oracle's binary codes."""
    codes, flags, _alpha, beta = oracle.binary_codes(p.w)
    g = to_np(gamma)[0]
    check_rel([g], [beta], SCALE_RTOL, "beta")
    got = to_np(packed)
    codes_gpu, bad = oracle.unpack(got, p.K, LAYOUT)
    assert bad == 0
    assert check_codes(codes_gpu, codes, flags, "codes") == 0 or g != beta
    assert np.array_equal(oracle.pack(codes_gpu, LAYOUT), got), "layout or padding differs"
    return codes_gpu


PACK_CASES = [(256, 256, "f32"), (37, 1000, "bf16"), (5, 17, "f32"), (3, 1, "f32"),
              (64, 130, "f32"), (129, 4099, "bf16"), (1, 65, "bf16")]


@pytest.mark.parametrize("N,K,dtype", PACK_CASES)
def test_pack_1bit_parity(bl, N, K, dtype):
    banner(f"pack 1bit N={N} K={K} {dtype}")
    p = synth.make_problem(M=1, N=N, K=K, seed=700 + N + K, dtype=dtype)
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, dtype == "bf16"), LAYOUT, SCHEME)
    torch.cuda.synchronize()
    assert packed.shape[1] == oracle.row_bytes(K, LAYOUT)
    check_packed(bl, packed, gamma, p)


def pipeline(bl, p, out_dtype):
    bf = p.dtype == "bf16"
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, bf), LAYOUT, SCHEME)
    xq, scale = bl.bitlinear_quant_acts(dev(p.x_store, bf))
    y, acc = bl.bitlinear_forward(xq, scale, packed, gamma, p.N, p.K, LAYOUT, out_dtype,
                                  acc=True)
    torch.cuda.synchronize()
    return packed, gamma, xq, scale, y, acc


FWD_CASES = [
    # decode product: one and several tokens, ragged K, two row groups (N >= 8192)
    (1, 256, 256), (3, 100, 1000), (5, 33, 17), (16, 300, 4099), (16, 8200, 64),
    # tiled GEMM: edge tiles, ragged K, several k-tiles
    (17, 64, 130), (300, 520, 264), (40, 1000, 333), (257, 700, 5000),
    # whole tiles over rows with padding codes (K = 976 in 1024-code rows): the
    # unguarded interior path must not run there (regression)
    (183, 478, 976), (256, 128, 976),
    # long rows: two wave groups split the k-tiles (no padding: unguarded
    # whole tiles; padding: guarded)
    (140, 333, 8192), (140, 200, 9000),
    # at most one round of 64 x 64 tiles over 32 k-tiles (launched as 32 x 128
    # tiles of the same area): split k-tiles on whole rows
    (200, 1000, 4096),
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", FWD_CASES)
def test_forward_1bit_parity(bl, M, N, K, out_dtype):
    banner(f"forward 1bit M={M} N={N} K={K} {out_dtype}")
    p = synth.make_problem(M=M, N=N, K=K, seed=800 + M + N + K, dtype="bf16",
                           outlier_frac=0.01)
    packed, gamma, xq, scale, y, acc = pipeline(bl, p, out_dtype)
    ref = oracle.forward(p.w, p.x, LAYOUT, SCHEME)
    codes_gpu = check_packed(bl, packed, gamma, p)
    check_codes(to_np(xq), ref["xq"], ref["xflags"], "xq")
    assert np.array_equal(to_np(scale), ref["scale"])
    ex = excluded_acc_mask(to_np(xq) != ref["xq"], codes_gpu != ref["codes"])
    assert np.array_equal(to_np(acc)[~ex], ref["acc"][~ex])
    if out_dtype == torch.float32:
        check_y_f32(to_np(y)[~ex], ref["y64"][~ex])
    else:
        check_y_bf16(y_bits(y)[~ex], ref["y64"][~ex])


def test_prefill_1bit_full_size_sampled(bl):
    """M=2048, K=4096, N=11008 (the one-launch pair of tile shapes): beta and
    every code compared; accumulators and bf16 outputs on 26 token rows."""
    banner("prefill full 1bit")
    p = synth.workload("prefill")
    packed, gamma, xq, scale, y, acc = pipeline(bl, p, torch.bfloat16)
    codes_gpu = check_packed(bl, packed, gamma, p)
    xq_ref, s_ref, xflags = oracle.quant_acts(p.x)
    check_codes(to_np(xq), xq_ref, xflags, "xq")
    rows = np.concatenate([np.random.default_rng(1).choice(p.M, 24, replace=False),
                           [0, p.M - 1]])
    acc_ref = oracle.int_product(xq_ref[rows], codes_gpu)
    assert np.array_equal(to_np(acc)[rows], acc_ref)
    y64 = oracle.epilogue(acc_ref, to_np(gamma)[0], s_ref[rows])
    check_y_bf16(y_bits(y)[rows], y64)


FUSED_CASES = [(1, 256, 256, "f32"), (2, 100, 1000, "bf16"), (3, 33, 17, "f32"),
               (4, 300, 9001, "bf16"), (1, 16400, 160, "bf16"), (3, 12000, 4096, "bf16"),
               (4, 9000, 4096, "f32"), (2, 20000, 512, "bf16"), (3, 33000, 300, "f32"),
               (1, 11008, 4096, "bf16"), (1, 300, 9001, "f32")]


@pytest.mark.parametrize("M,N,K,dtype", FUSED_CASES)
def test_fused_1bit_parity(bl, M, N, K, dtype):
    banner(f"fused 1bit M={M} N={N} K={K} {dtype}")
    p = synth.make_problem(M=M, N=N, K=K, seed=900 + M + N + K, dtype=dtype, outlier_frac=0.01)
    bf = dtype == "bf16"
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, bf), LAYOUT, SCHEME)
    y, acc = bl.bitlinear_linear(dev(p.x_store, bf), packed, gamma, N, LAYOUT, acc=True)
    torch.cuda.synchronize()
    ref = oracle.forward(p.w, p.x, LAYOUT, SCHEME)
    codes_gpu = check_packed(bl, packed, gamma, p)
    # the fused quantiser takes every activation code in the same fp32 steps
    # as the oracle (also inside the boundary band), so the sums are exact
    assert np.array_equal(codes_gpu, ref["codes"])
    assert np.array_equal(to_np(acc), ref["acc"])
    check_y_f32(to_np(y), ref["y64"])


def test_decode_1bit_full(bl):
    """The decode workload (M=1, 4096 x 4096, bf16 with outliers), fused step."""
    banner("decode full 1bit")
    p = synth.workload("decode")
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, True), LAYOUT, SCHEME)
    y, acc = bl.bitlinear_linear(dev(p.x_store, True), packed, gamma, p.N, LAYOUT, acc=True)
    torch.cuda.synchronize()
    assert packed.numel() == 4096 * 4096 // 8
    ref = oracle.forward(p.w, p.x, LAYOUT, SCHEME)
    codes_gpu = check_packed(bl, packed, gamma, p)
    ex = excluded_acc_mask(np.zeros_like(ref["xq"], bool), codes_gpu != ref["codes"])
    assert np.array_equal(to_np(acc)[~ex], ref["acc"][~ex])
    check_y_f32(to_np(y)[~ex], ref["y64"][~ex])


@pytest.mark.parametrize("M", [2, 24])
def test_segmented_1bit(bl, M):
    """Three stacked 1-bit matrices with their own beta: the fused step (M=2)
    and quantise + segmented product (M=24, the GEMM)."""
    segs, K = (300, 40, 1000), 520
    banner(f"segmented 1bit M={M} segs={segs} K={K}")
    rng = np.random.default_rng(M)
    codes = [np.where(rng.random((n, K)) < 0.5, -1, 1).astype(np.int8) for n in segs]
    betas = np.zeros(4, np.float32)
    betas[:3] = rng.uniform(0.005, 0.05, size=3)
    packed = dev(np.concatenate([oracle.pack(c, LAYOUT) for c in codes], axis=0))
    p = synth.make_problem(M=M, N=1, K=K, seed=77 + M, dtype="bf16")
    x = dev(p.x_store, True)
    if M <= 4:
        y, acc = bl.bitlinear_linear_segmented(x, packed, dev(betas), segs, LAYOUT, acc=True)
    else:
        xq, scale = bl.bitlinear_quant_acts(x)
        y, acc = bl.bitlinear_forward_segmented(xq, scale, packed, dev(betas), segs, K, LAYOUT,
                                                acc=True)
    torch.cuda.synchronize()
    xq_ref, s_ref, _ = oracle.quant_acts(p.x)  # same fp32 steps on both sides
    acc_ref = oracle.int_product(xq_ref, np.concatenate(codes, axis=0))
    assert np.array_equal(to_np(acc), acc_ref)
    cols, parts = 0, []
    for c, b in zip(codes, betas):
        parts.append(oracle.epilogue(acc_ref[:, cols:cols + c.shape[0]], b, s_ref))
        cols += c.shape[0]
    check_y_f32(to_np(y), np.concatenate(parts, axis=1))
