"""GPU parity of the lookup-table decode GEMV (bitlinear_forward_lut, base-3
codes, one token) against the oracle and against the in-register decode of
bitlinear_forward: INT32 accumulators bit-exact, y within the output
tolerance."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import check_y_bf16, check_y_f32, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# (N, K): one and several 5120-code chunks, ragged N and K, a group straddling K
LUT_CASES = [(256, 256), (37, 1001), (4096, 4096), (100, 5120), (64, 5121), (300, 11008), (1, 7)]


@pytest.mark.parametrize("N,K", LUT_CASES)
def test_forward_lut_parity(bl, N, K):
    print(f"[case] forward_lut N={N} K={K}", flush=True)
    rng = np.random.default_rng(N * 13 + K)
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    xq = rng.integers(-127, 128, size=(1, K)).astype(np.int8)
    scale = np.array([rng.uniform(0.5, 30.0)], np.float32)
    gamma = np.float32(0.0213)
    packed = dev(oracle.pack(codes, "base3"))
    g = torch.tensor([gamma, 0, 0, 0], dtype=torch.float32, device="cuda")
    acc_ref = oracle.int_product(xq, codes)
    y64 = oracle.epilogue(acc_ref, gamma, scale)
    for ydt in (torch.float32, torch.bfloat16):
        y, acc = bl.bitlinear_forward_lut(dev(xq), dev(scale), packed, g, N, K, ydt, acc=True)
        y2, acc2 = bl.bitlinear_forward(dev(xq), dev(scale), packed, g, N, K, "base3", ydt, acc=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(acc), acc_ref), "INT32 accumulators differ"
        assert torch.equal(acc, acc2)
        if ydt == torch.float32:
            check_y_f32(to_np(y), y64)
        else:
            check_y_bf16(to_np(y.view(torch.int16)).view(np.uint16), y64)


def test_forward_lut_decode_workload(bl):
    """The decode workload (4096 x 4096 bf16 weights, one token with
    outliers) through pack -> quant_acts -> lookup GEMV, against the oracle's
    whole forward pass."""
    p = synth.workload("decode")
    print(f"[case] forward_lut decode N={p.N} K={p.K}", flush=True)
    W = torch.from_numpy(p.w_store.view(np.int16)).cuda().view(torch.bfloat16)
    x = torch.from_numpy(p.x_store.view(np.int16)).cuda().view(torch.bfloat16)
    packed, gamma = bl.bitlinear_pack_weights(W, "base3")
    xq, scale = bl.bitlinear_quant_acts(x)
    y, acc = bl.bitlinear_forward_lut(xq, scale, packed, gamma, p.N, p.K, acc=True)
    torch.cuda.synchronize()
    ref = oracle.forward(p.w, p.x, "base3")
    assert not ref["wflags"].any() and not ref["xflags"].any()
    assert np.array_equal(to_np(acc), ref["acc"])
    check_y_f32(to_np(y), ref["y64"])
