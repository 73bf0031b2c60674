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


def packed_problem(bl, M, N, K, seed, scheme="ternary", layout="2bit"):
    p = synth.make_problem(M=M, N=N, K=K, seed=seed, dtype="bf16", grad_std=1e-3)
    packed, gamma = bl.bitlinear_pack_weights(dev(p.w_store, True), layout, scheme)
    torch.cuda.synchronize()
    codes, bad = oracle.unpack(to_np(packed), K, layout)  # the codes the GPU will use
    assert bad == 0
    return p, packed, gamma, codes, float(to_np(gamma)[0])


def check_grad_x(bl, p, packed, gamma, codes, g, layout, rows=None):
    gx = to_np(bl.bitlinear_backward_input(dev(p.grad_y_store, True), packed, gamma, p.K, layout))
    gy = p.grad_y if rows is None else np.ascontiguousarray(p.grad_y[rows])
    if rows is not None:
        gx = gx[rows]
    ref = oracle.ste_grad_x(gy, codes, g)
    abs_sum = (np.abs(gy.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    return check_sum(gx, ref, abs_sum, p.N, f"grad_x ({layout})")


BWD_CASES = [
    (64, 64, 64), (300, 520, 264), (257, 1024, 136), (33, 8, 1000), (512, 776, 520),
    (17, 264, 2056),
]


SCHEME = {"2bit": "ternary", "base3": "ternary", "1bit": "binary"}


@pytest.mark.parametrize("layout", ["2bit", "base3", "1bit"])
@pytest.mark.parametrize("M,N,K", BWD_CASES)
def test_backward_input_parity(bl, M, N, K, layout):
    """grad_x straight from the forward's packed rows in each layout (ternary
    codes for 2-bit and base-3, binary codes for the 1-bit layout)."""
    banner(f"backward_input {layout} M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=500 + M + N + K,
                                                scheme=SCHEME[layout], layout=layout)
    check_grad_x(bl, p, packed, gamma, codes, g, layout)


@pytest.mark.parametrize("M,N,K", [c for c in BWD_CASES if c[2] % 8 == 0])
def test_backward_weight_parity(bl, M, N, K):
    banner(f"backward_weight M={M} N={N} K={K}")
    p = synth.make_problem(M=M, N=N, K=K, seed=600 + M + N + K, dtype="bf16", grad_std=1e-3)
    gw = bl.bitlinear_backward_weight(dev(p.grad_y_store, True), dev(p.x_store, True))
    torch.cuda.synchronize()
    ref = oracle.ste_grad_w(p.grad_y, p.x)
    abs_sum = np.abs(p.grad_y.astype(np.float64)).T @ np.abs(p.x.astype(np.float64))
    check_sum(to_np(gw), ref, abs_sum, M, "grad_w")


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 520, 264), (33, 8, 1000), (17, 264, 2056),
                                   (6, 16, 24)])
def test_backward_weight_fp32(bl, M, N, K):
    """fp32 grad_y and x: six piece products per term, summed in fp32 (6M
    terms), with the three dropped pairs under 2^-20 (= 16 u) of each
    product: bound (6M + 16) u per unit of the sum of |terms|. At M = 6 that
    is ~3e-6 of it, against 2^-14 for a lost lo piece or a lost pair."""
    banner(f"backward_weight fp32 M={M} N={N} K={K}")
    p = synth.make_problem(M=M, N=N, K=K, seed=700 + M + N + K, dtype="f32", grad_std=1e-3)
    gy = np.ascontiguousarray(p.grad_y, np.float32)
    x = np.ascontiguousarray(p.x, np.float32)
    gw = to_np(bl.bitlinear_backward_weight(dev(gy), dev(x)))
    ref = oracle.ste_grad_w(gy, x)
    abs_sum = np.abs(gy.astype(np.float64)).T @ np.abs(x.astype(np.float64))
    check_sum(gw, ref, abs_sum, 6 * M + 16, "grad_w fp32")


def test_backward_weight_fp32_wide_range(bl):
    """Both operands with full 24-bit significands over exponents 2^-50 .. 2^20
    and both signs (products stay far from fp32's range limits)."""
    M, N, K = 8, 64, 96
    banner(f"backward_weight fp32 wide range M={M} N={N} K={K}")
    rng = np.random.default_rng(13)

    def wide(shape):
        mant = 1.0 + rng.integers(0, 1 << 23, size=shape) / float(1 << 23)
        expo = rng.integers(-50, 21, size=shape)
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        return (sign * mant * np.exp2(expo)).astype(np.float32)

    gy, x = wide((M, N)), wide((M, K))
    gw = to_np(bl.bitlinear_backward_weight(dev(gy), dev(x)))
    ref = oracle.ste_grad_w(gy, x)
    abs_sum = np.abs(gy.astype(np.float64)).T @ np.abs(x.astype(np.float64))
    check_sum(gw, ref, abs_sum, 6 * M + 16, "grad_w fp32 wide range")


@pytest.mark.parametrize("layout", ["2bit", "base3", "1bit"])
@pytest.mark.parametrize("K", [1001, 5, 255, 261, 1281])
def test_backward_input_ragged_k(bl, layout, K):
    """K not a multiple of the tile width nor of a layout's code group (16-code
    words of the 2-bit layout, 5-code bytes of base-3, 32-code words of 1-bit):
    the rows end inside a group, and for base-3 a thread's 32 codes start
    inside a byte (K = 261, 1281 put a tile edge mid-byte)."""
    M, N = 40, 96
    banner(f"backward_input ragged K {layout} M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=77 + K,
                                                scheme=SCHEME[layout], layout=layout)
    check_grad_x(bl, p, packed, gamma, codes, g, layout)


@pytest.mark.parametrize("layout", ["2bit", "base3", "1bit"])
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 520, 264), (33, 8, 1000), (17, 264, 2056)])
def test_backward_input_fp32_grad(bl, M, N, K, layout):
    """fp32 grad_y: each value is split exactly into three bf16 pieces and the
    3N products of the pieces with the codes are summed in fp32, so the bound
    is the fp32 summation bound over 3N terms (|hi| + |mid| + |lo| = |g|, so
    the sum of |terms| is unchanged). At N = 8 the bound is ~1.4e-6 of the sum
    of |terms|: losing the low piece (2^-16 relative) would fail it."""
    banner(f"backward_input fp32 grad_y {layout} M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=900 + M + N + K,
                                                scheme=SCHEME[layout], layout=layout)
    gy = np.ascontiguousarray(p.grad_y, np.float32)
    gx = to_np(bl.bitlinear_backward_input(dev(gy), packed, gamma, K, layout))
    ref = oracle.ste_grad_x(gy, codes, g)
    abs_sum = (np.abs(gy.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(gx, ref, abs_sum, 3 * N, f"grad_x fp32 ({layout})")


def test_backward_input_fp32_wide_range(bl):
    """fp32 grad_y with full 24-bit significands over exponents 2^-100 .. 2^30
    and both signs, against codes of all +1 in a few columns (so each output is
    a plain sum whose low bits come from the mid and lo pieces)."""
    M, N, K = 96, 16, 64
    banner(f"backward_input fp32 wide range M={M} N={N} K={K}")
    rng = np.random.default_rng(12)
    mant = 1.0 + rng.integers(0, 1 << 23, size=(M, N)) / float(1 << 23)
    expo = rng.integers(-100, 31, size=(M, N))
    gy = (np.where(rng.random((M, N)) < 0.5, -1.0, 1.0) * mant * np.exp2(expo)).astype(np.float32)
    codes = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    codes[:, :4] = 1
    packed_np = oracle.pack(codes, "2bit")
    g = 1.0
    gamma = torch.tensor([g], dtype=torch.float32, device="cuda")
    gx = to_np(bl.bitlinear_backward_input(dev(gy), dev(packed_np), gamma, K, "2bit"))
    ref = oracle.ste_grad_x(gy, codes, g)
    abs_sum = np.abs(gy.astype(np.float64)) @ np.abs(codes.astype(np.float64))
    check_sum(gx, ref, abs_sum, 3 * N, "grad_x fp32 wide range")


def test_backward_input_binary_codes(bl):
    """1-bit codes (+-1 in the 2-bit container) through the 2-bit product."""
    M, N, K = 128, 256, 320
    banner(f"backward_input binary M={M} N={N} K={K}")
    p, packed, gamma, codes, g = packed_problem(bl, M, N, K, seed=88, scheme="binary")
    assert set(np.unique(codes)) <= {-1, 1}
    check_grad_x(bl, p, packed, gamma, codes, g, "2bit")


@pytest.mark.parametrize("layout", ["base3", "1bit"])
def test_backward_input_every_code_pattern(bl, layout):
    """Every byte value of the layout in every position of a row: base-3 bytes
    0..242 and 1-bit bytes 0..255, so every trit or bit place of every byte
    (and every offset of a 32-code run inside base-3 bytes) meets the
    expansion to bf16. The codes are the oracle's unpacking of the bytes."""
    K = {"base3": 243 * 5, "1bit": 256 * 8}[layout]
    rb = bl.bitlinear_packed_row_bytes(K, layout)
    N, M = 64, 48
    banner(f"backward_input every code pattern {layout} M={M} N={N} K={K}")
    rng = np.random.default_rng(4)
    nvals = 243 if layout == "base3" else 256
    packed_np = np.zeros((N, rb), np.uint8)
    for n in range(N):
        packed_np[n, :nvals] = np.roll(np.arange(nvals, dtype=np.uint8), 7 * n)
    if layout == "base3":
        packed_np[:, nvals:] = 121  # five zero codes
    codes, bad = oracle.unpack(packed_np, K, layout)
    assert bad == 0
    p = synth.make_problem(M=M, N=N, K=K, seed=41, dtype="bf16", grad_std=1e-3)
    g = 0.75
    gamma = torch.tensor([g], dtype=torch.float32, device="cuda")
    gx = to_np(bl.bitlinear_backward_input(dev(p.grad_y_store, True), dev(packed_np), gamma, K,
                                           layout))
    ref = oracle.ste_grad_x(p.grad_y, codes, g)
    abs_sum = (np.abs(p.grad_y.astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(gx, ref, abs_sum, N, f"grad_x ({layout})")


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
    # the same with fp32 operands
    gx.fill_(7.0)
    gw.fill_(7.0)
    assert lib.bitlinear_backward_input(P(dummy), 0, P(packed), 0, P(gamma), 5, 0, 24, P(gx), s) == 0
    assert lib.bitlinear_backward_weight(P(dummy), P(dummy), 0, 0, 16, 24, P(gw), s) == 0
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
    gw = to_np(bl.bitlinear_backward_weight(gy, dev(p.x_store, True)))
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(M, 6, replace=False))
    check_grad_x(bl, p, packed, gamma, codes, g, "2bit", rows=rows)
    cols = np.sort(rng.choice(N, 6, replace=False))
    ref = oracle.ste_grad_w(np.ascontiguousarray(p.grad_y[:, cols]), p.x)
    abs_sum = np.abs(p.grad_y[:, cols].astype(np.float64)).T @ np.abs(p.x.astype(np.float64))
    check_sum(gw[cols], ref, abs_sum, M, "grad_w rows")


@pytest.mark.parametrize("variant", ["base3", "1bit", "fp32_grad_y"])
def test_training_shapes_other_inputs(bl, variant):
    """The benchmark's grad_x beside the training step, at 4096 x 4096 x 4096:
    from the base-3 and 1-bit packed rows of the same weights, and from fp32
    grad_y against the 2-bit rows. Sampled rows against the oracle (each a
    full contraction of length 4096)."""
    t = synth.workload("train")
    M, N, K = t.M, t.N, t.K
    banner(f"backward training shapes {variant} M={M} N={N} K={K}")
    layout = {"base3": "base3", "1bit": "1bit", "fp32_grad_y": "2bit"}[variant]
    scheme = "binary" if layout == "1bit" else "ternary"
    packed, gamma = bl.bitlinear_pack_weights(dev(t.w_store, True), layout, scheme)
    torch.cuda.synchronize()
    codes, bad = oracle.unpack(to_np(packed), K, layout)
    assert bad == 0
    g = float(to_np(gamma)[0])
    if variant == "fp32_grad_y":
        gy = np.ascontiguousarray(t.grad_y, np.float32)  # bf16 values widened, as the benchmark does
        gx = to_np(bl.bitlinear_backward_input(dev(gy), packed, gamma, K, layout))
        n_terms = 3 * N
    else:
        gy = t.grad_y
        gx = to_np(bl.bitlinear_backward_input(dev(t.grad_y_store, True), packed, gamma, K, layout))
        n_terms = N
    rows = np.sort(np.random.default_rng(6).choice(M, 6, replace=False))
    ref = oracle.ste_grad_x(np.ascontiguousarray(gy[rows], np.float32), codes, g)
    abs_sum = (np.abs(gy[rows].astype(np.float64)) @ np.abs(codes.astype(np.float64))) * g
    check_sum(gx[rows], ref, abs_sum, n_terms, f"grad_x rows ({variant})")


def test_training_shapes_weight_fp32(bl):
    """The benchmark's fp32 grad_W beside the training step (bf16 grad_y and x
    widened to fp32, 4096 x 4096 x 4096): sampled rows of grad_W."""
    t = synth.workload("train")
    M, N, K = t.M, t.N, t.K
    banner(f"backward_weight fp32 training shapes M={M} N={N} K={K}")
    gy = np.ascontiguousarray(t.grad_y, np.float32)
    x = np.ascontiguousarray(t.x, np.float32)
    gw = to_np(bl.bitlinear_backward_weight(dev(gy), dev(x)))
    cols = np.sort(np.random.default_rng(7).choice(N, 6, replace=False))
    ref = oracle.ste_grad_w(np.ascontiguousarray(gy[:, cols]), x)
    abs_sum = np.abs(gy[:, cols].astype(np.float64)).T @ np.abs(x.astype(np.float64))
    check_sum(gw[cols], ref, abs_sum, 6 * M + 16, "grad_w fp32 rows")
