"""The largest contraction the forward calls accept: K = floor((2^31 - 1) / 127),
where |acc| = 127 K = 2,147,483,640 is one step from INT32 overflow.

The case has a closed form, so no oracle run is needed (and none of the
oracle's arithmetic is re-typed here): every |w| is bf16(0.02), so gamma is
exactly that value and every code is +-1 (row n has sign (-1)^n); every
activation is +-1.0 (token m has sign (-1)^m), so s_m = 1 and every INT8 code
is +-127. Hence acc[m, n] = (-1)^(m+n) * 127 * K exactly, and
y[m, n] = acc * gamma * 1 / 127 = (-1)^(m+n) * K * gamma.

The extreme is checked through every product path: the fused decode step
(1 and 2 tokens), the decode product (5 tokens), the tiled GEMM (17 tokens)
and, for base-3, the lookup-table product."""
import numpy as np
import pytest
import torch

from parity_util import check_y_f32, to_np

pytestmark = pytest.mark.gpu

K_MAX = (2 ** 31 - 1) // 127
N = 16


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def signs(n):
    return np.where(np.arange(n) % 2 == 0, 1, -1).astype(np.int64)


def expected(M, gamma):
    acc = np.outer(signs(M), signs(N)) * (127 * K_MAX)
    assert np.abs(acc).max() <= 2 ** 31 - 1
    return acc.astype(np.int32), acc.astype(np.float64) * np.float64(gamma) / 127.0


@pytest.fixture(scope="module", params=["2bit", "base3"])
def packed_max(bl, request):
    layout = request.param
    print(f"[case] max-K pack {layout} N={N} K={K_MAX}", flush=True)
    W = torch.full((N, K_MAX), 0.02, dtype=torch.bfloat16, device="cuda")
    W[1::2] = -W[1::2]
    packed, gamma = bl.bitlinear_pack_weights(W, layout)
    del W
    torch.cuda.synchronize()
    g = float(to_np(gamma)[0])
    # the mean of equal magnitudes is that magnitude
    assert g == float(torch.tensor(0.02, dtype=torch.bfloat16).float())
    return layout, packed, gamma, g


def x_tokens(M):
    x = torch.ones((M, K_MAX), dtype=torch.bfloat16, device="cuda")
    x[1::2] = -1.0
    return x


@pytest.mark.parametrize("M", [1, 2])
def test_max_k_fused(bl, packed_max, M):
    layout, packed, gamma, g = packed_max
    print(f"[case] max-K fused {layout} M={M}", flush=True)
    y, acc = bl.bitlinear_linear(x_tokens(M), packed, gamma, N, layout, acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = expected(M, g)
    assert np.array_equal(to_np(acc), acc_ref)
    check_y_f32(to_np(y), y_ref)


@pytest.mark.parametrize("M", [5, 17])
def test_max_k_quantise_then_multiply(bl, packed_max, M):
    layout, packed, gamma, g = packed_max
    print(f"[case] max-K two-launch {layout} M={M}", flush=True)
    xq, scale = bl.bitlinear_quant_acts(x_tokens(M))
    torch.cuda.synchronize()
    assert torch.all(scale == 1.0)
    assert torch.equal(xq[0::2], torch.full_like(xq[0::2], 127))
    assert torch.equal(xq[1::2], torch.full_like(xq[1::2], -127))
    y, acc = bl.bitlinear_forward(xq, scale, packed, gamma, N, K_MAX, layout, acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = expected(M, g)
    assert np.array_equal(to_np(acc), acc_ref)
    check_y_f32(to_np(y), y_ref)


def test_max_k_lookup_table(bl, packed_max):
    layout, packed, gamma, g = packed_max
    if layout != "base3":
        pytest.skip("the lookup-table product reads base-3 codes only")
    print("[case] max-K lookup table", flush=True)
    xq, scale = bl.bitlinear_quant_acts(x_tokens(1))
    y, acc = bl.bitlinear_forward_lut(xq, scale, packed, gamma, N, K_MAX, acc=True)
    torch.cuda.synchronize()
    acc_ref, y_ref = expected(1, g)
    assert np.array_equal(to_np(acc), acc_ref)
    check_y_f32(to_np(y), y_ref)

