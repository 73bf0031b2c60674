"""GPU parity of the straight-through-estimator backward products
(bitlinear_backward_input / bitlinear_backward_weight) against the oracle's
fp64 sums, on the same seeded inputs and the same codes.

Bar (derived from the arithmetic): every product term is exact in fp32 (bf16 x
bf16 has 16 significant bits; bf16 x {-1, 0, +1} is a bf16 value), so the only
error is the rounding of the fp32 additions (in any order, inside or between
matrix-core instructions) and of the final scaling by gamma. For n additions
|err| <= n * u * S with u = 2^-24 and S = sum of |terms|; scaling adds u |ref|.
The test allows 1.01 x that worst case and reports how much of it is used."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import to_np

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def banner(msg):
    print(f"[case] {msg}", flush=True)


def check_sum(got: np.ndarray, ref: np.ndarray, abs_sum: np.ndarray, n: int, what: str) -> float:
    bound = 1.01 * (n * U * abs_sum + U * np.abs(ref)) + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the fp32 summation bound"
    return worst


def packed_problem(bl, M, N, K, seed, scheme="ternary"):
    p = synth.make_problem(M=M, N=N, K=K, seed=seed, dtype="bf16", grad_std=1e-3)
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, True), "2bit", scheme)
    torch.cuda.synchronize()
    codes, bad = oracle.unpack(to_np(packed), K, "2bit")  # the codes the GPU will use
    assert bad == 0
    return p, packed, gamma, codes, float(to_np(gamma)[0])


BWD_CASES = [
    (64, 64, 64), (300, 520, 264), (257, 1024, 136), (33, 8, 1000), (512, 776, 520),
    (17, 264, 2056),
]


@pytest.mark.parametrize("M,N,K", BWD_CASES)
def test_backward_input_parity(bl, M, N, K):
    banner(f"backward_input M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=500 + M + N + K)
    gx = bl.bitlinear_backward_input(dev(p.grad_y_store, True), packed, gamma, K)
    torch.cuda.synchronize()
    ref = oracle.ste_grad_x(p.grad_y, codes, g)
    abs_sum = (np.abs(p.grad_y.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(to_np(gx), ref, abs_sum, N, "grad_x")


@pytest.mark.parametrize("M,N,K", [c for c in BWD_CASES if c[2] % 8 == 0])
def test_backward_weight_parity(bl, M, N, K):
    banner(f"backward_weight M={M} N={N} K={K}")
    p = synth.make_problem(M=M, N=N, K=K, seed=600 + M + N + K, dtype="bf16", grad_std=1e-3)
    gw = bl.bitlinear_backward_weight(dev(p.grad_y_store, True), dev(p.x_store, True))
    torch.cuda.synchronize()
    ref = oracle.ste_grad_w(p.grad_y, p.x)
    abs_sum = np.abs(p.grad_y.astype(np.float64)).T @ np.abs(p.x.astype(np.float64))
    check_sum(to_np(gw), ref, abs_sum, M, "grad_w")


def test_backward_input_ragged_k(bl):
    """K not a multiple of 8 (the packed rows end inside a 16-code group)."""
    M, N, K = 40, 96, 1001
    banner(f"backward_input ragged K M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=77)
    gx = bl.bitlinear_backward_input(dev(p.grad_y_store, True), packed, gamma, K)
    torch.cuda.synchronize()
    ref = oracle.ste_grad_x(p.grad_y, codes, g)
    abs_sum = (np.abs(p.grad_y.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(to_np(gx), ref, abs_sum, N, "grad_x")


def test_backward_input_binary_codes(bl):
    """1-bit codes (+-1 in the 2-bit container) through the same product."""
    M, N, K = 128, 256, 320
    banner(f"backward_input binary M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=88, scheme="binary")
    assert set(np.unique(codes)) <= {-1, 1}
    gx = bl.bitlinear_backward_input(dev(p.grad_y_store, True), packed, gamma, K)
    torch.cuda.synchronize()
    ref = oracle.ste_grad_x(p.grad_y, codes, g)
    abs_sum = (np.abs(p.grad_y.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(to_np(gx), ref, abs_sum, N, "grad_x")


def test_backward_empty_sums_write_zeros(bl):
    """An empty contraction (N = 0 for grad_x, M = 0 for grad_w) is a sum of
    nothing: the outputs are zeros."""
    banner("backward empty sums")
    lib = bl.library()
    dummy = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    gamma = torch.ones(4, dtype=torch.float32, device="cuda")
    packed = torch.zeros(16, dtype=torch.uint8, device="cuda")
    gx = torch.full((5, 24), 7.0, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    assert lib.bitlinear_backward_input(P(dummy), 1, P(packed), 0, P(gamma), 5, 0, 24, P(gx), s) == 0
    gw = torch.full((16, 24), 7.0, device="cuda")
    assert lib.bitlinear_backward_weight(P(dummy), P(dummy), 1, 0, 16, 24, P(gw), s) == 0
    torch.cuda.synchronize()
    assert not gx.any() and not gw.any()


def test_training_shapes_sampled(bl):
    """The 4096 x 4096 x 4096 training step shapes, in the launch configuration
    the benchmark times: sampled rows of grad_x and sampled rows of grad_w
    against the oracle (each is a full contraction of length 4096)."""
    cfg = synth.WORKLOADS["train"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    banner(f"backward training shapes M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=cfg["seed"])
    gy = dev(p.grad_y_store, True)
    gx = to_np(bl.bitlinear_backward_input(gy, packed, gamma, K))
    gw = to_np(bl.bitlinear_backward_weight(gy, dev(p.x_store, True)))
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(M, 6, replace=False))
    ref = oracle.ste_grad_x(p.grad_y[rows], codes, g)
    abs_sum = (np.abs(p.grad_y[rows].astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(gx[rows], ref, abs_sum, N, "grad_x rows")
    cols = np.sort(rng.choice(N, 6, replace=False))
    ref = oracle.ste_grad_w(np.ascontiguousarray(p.grad_y[:, cols]), p.x)
    abs_sum = np.abs(p.grad_y[:, cols].astype(np.float64)).T @ np.abs(p.x.astype(np.float64))
    check_sum(gw[cols], ref, abs_sum, M, "grad_w rows")
