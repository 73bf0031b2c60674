"""GPU parity of the stacked-matrix calls (bitlinear_forward_segmented /
bitlinear_linear_segmented): several row segments, each with its own gamma,
in one launch. Per segment the result must be that of the oracle on the
segment alone: INT32 accumulators bit-exact, y within the output tolerance."""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth
from parity_util import check_codes, check_y_bf16, check_y_f32, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def banner(msg):
    print(f"[case] {msg}", flush=True)


def stacked(segs, K, layout, seed):
    """Random codes per segment, packed one after the other; distinct gammas."""
    rng = np.random.default_rng(seed)
    codes = [rng.integers(-1, 2, size=(n, K)).astype(np.int8) for n in segs]
    gammas = rng.uniform(0.005, 0.05, size=len(segs)).astype(np.float32)
    packed = np.concatenate([oracle.pack(c, layout) for c in codes], axis=0)
    return codes, gammas, packed


def gpu_gammas(gammas):
    g = np.zeros(max(4, (len(gammas) + 3) // 4 * 4), np.float32)
    g[:len(gammas)] = gammas
    return dev(g)


def ref_y(acc_ref, codes, gammas, scale):
    cols, y = 0, []
    for c, g in zip(codes, gammas):
        n = c.shape[0]
        y.append(oracle.epilogue(acc_ref[:, cols:cols + n], g, scale))
        cols += n
    return np.concatenate(y, axis=1)


FWD_CASES = [
    # (M, segments, K): skinny (M <= 16), tiled GEMM (M > 16), ragged rows and K
    (1, (64, 48, 80), 256), (4, (100, 36, 120), 200), (16, (16, 16, 16), 1000),
    (9, (3, 5, 7, 11, 13, 17, 19, 23), 96), (40, (100, 36, 120), 200), (300, (64, 48, 80), 333),
    # long rows in the GEMM: two wave groups split the k-tiles (ragged K: the
    # guarded path; K = 8192: whole tiles unguarded)
    (130, (600, 400, 1000), 9000), (200, (520, 1000, 300), 8192),
]


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("M,segs,K", FWD_CASES)
def test_forward_segmented_parity(bl, layout, M, segs, K):
    banner(f"forward_segmented {layout} M={M} segs={segs} K={K}")
    codes, gammas, packed = stacked(segs, K, layout, seed=M * 31 + K + len(segs))
    rng = np.random.default_rng(K)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    scale = rng.uniform(0.5, 30.0, size=M).astype(np.float32)
    acc_ref = oracle.int_product(xq, np.concatenate(codes, axis=0))
    y64 = ref_y(acc_ref, codes, gammas, scale)
    g = gpu_gammas(gammas)
    for ydt in (torch.float32, torch.bfloat16):
        y, acc = bl.bitlinear_forward_segmented(dev(xq), dev(scale), dev(packed), g, segs, K,
                                                layout, ydt, acc=True)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(acc), acc_ref), "INT32 accumulators differ"
        if ydt == torch.float32:
            check_y_f32(to_np(y), y64)
        else:
            check_y_bf16(to_np(y.view(torch.int16)).view(np.uint16), y64)


def test_forward_segmented_split_launch(bl):
    """A prefill-sized stack (2-bit) runs as a main launch of 256 x 256 tiles
    plus a launch over the leftover columns; a segment boundary falls at the
    split, so the second launch must see the segment table shifted."""
    M, segs, K = 2048, (4096, 4096, 4096), 64
    banner(f"forward_segmented split M={M} segs={segs} K={K}")
    codes, gammas, packed = stacked(segs, K, "2bit", seed=5)
    rng = np.random.default_rng(6)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    scale = rng.uniform(0.5, 30.0, size=M).astype(np.float32)
    y, acc = bl.bitlinear_forward_segmented(dev(xq), dev(scale), dev(packed), gpu_gammas(gammas),
                                            segs, K, "2bit", torch.float32, acc=True)
    torch.cuda.synchronize()
    acc_ref = oracle.int_product(xq, np.concatenate(codes, axis=0))
    assert np.array_equal(to_np(acc), acc_ref)
    check_y_f32(to_np(y), ref_y(acc_ref, codes, gammas, scale))


def test_forward_segmented_one_segment_matches_plain(bl):
    M, N, K = 24, 200, 300
    codes, gammas, packed = stacked((N,), K, "2bit", seed=11)
    rng = np.random.default_rng(12)
    xq, scale = dev(rng.integers(-127, 128, size=(M, K)).astype(np.int8)), dev(
        rng.uniform(0.5, 30.0, size=M).astype(np.float32))
    g = gpu_gammas(gammas)
    a = bl.bitlinear_forward_segmented(xq, scale, dev(packed), g, (N,), K, "2bit")
    b = bl.bitlinear_forward(xq, scale, dev(packed), g[:1], N, K, "2bit")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("M", [1, 3, 4])
def test_linear_segmented_parity(bl, layout, M):
    """The fused decode step over Q, K, V-like segments, from bf16 x."""
    segs, K = (4096 // 8, 1024 // 8, 1024 // 8), 512
    banner(f"linear_segmented {layout} M={M} segs={segs} K={K}")
    codes, gammas, packed = stacked(segs, K, layout, seed=40 + M)
    p = synth.make_problem(M=M, N=1, K=K, seed=41 + M, dtype="bf16", outlier_frac=0.01)
    x = torch.from_numpy(p.x_store.view(np.int16)).cuda().view(torch.bfloat16)
    y, acc = bl.bitlinear_linear_segmented(x, dev(packed), gpu_gammas(gammas), segs, layout,
                                           torch.float32, acc=True)
    torch.cuda.synchronize()
    xq, scale, xflags = oracle.quant_acts(p.x)
    acc_ref = oracle.int_product(xq, np.concatenate(codes, axis=0))
    assert not xflags.any()
    assert np.array_equal(to_np(acc), acc_ref), "INT32 accumulators differ"
    check_y_f32(to_np(y), ref_y(acc_ref, codes, gammas, scale))


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("segs", [(4100, 1030, 3500), (8000, 4000, 4500), (20000, 9000, 4000)])
def test_linear_segmented_streaming(bl, layout, segs):
    """Fused decode of 3 tokens over stacks whose segment boundaries fall
    inside blocks: 8630 rows (540 tiles, more than the capped grid of two
    blocks per compute unit: blocks stream tiles), 16500 rows (two 16-row
    groups per block), 33000 rows (four); ragged segments, the last tile
    partly empty."""
    K = 1024
    M = 3
    banner(f"linear_segmented streaming {layout} M={M} segs={segs} K={K}")
    codes, gammas, packed = stacked(segs, K, layout, seed=77)
    p = synth.make_problem(M=M, N=1, K=K, seed=78, dtype="bf16", outlier_frac=0.01)
    x = torch.from_numpy(p.x_store.view(np.int16)).cuda().view(torch.bfloat16)
    y, acc = bl.bitlinear_linear_segmented(x, dev(packed), gpu_gammas(gammas), segs, layout,
                                           torch.float32, acc=True)
    torch.cuda.synchronize()
    xq, scale, _ = oracle.quant_acts(p.x)
    acc_ref = oracle.int_product(xq, np.concatenate(codes, axis=0))
    assert np.array_equal(to_np(acc), acc_ref), "INT32 accumulators differ"
    check_y_f32(to_np(y), ref_y(acc_ref, codes, gammas, scale))


@pytest.mark.parametrize("layout", ["2bit", "base3"])
def test_stacked_pack_end_to_end(bl, layout):
    """Q, K, V-like matrices packed one after the other into one buffer, each
    with its gamma written to consecutive floats, then one segmented launch,
    against the oracle's whole forward pass per matrix."""
    M, K, segs = 12, 320, (192, 64, 64)
    banner(f"stacked pack {layout} M={M} segs={segs} K={K}")
    probs = [synth.make_problem(M=M, N=n, K=K, seed=900 + i, dtype="bf16")
             for i, n in enumerate(segs)]
    x = probs[0].x_store  # one shared input
    rb = bl.bitlinear_packed_row_bytes(K, layout)
    packed = torch.empty((sum(segs), rb), dtype=torch.uint8, device="cuda")
    gammas = torch.zeros(4, dtype=torch.float32, device="cuda")
    r0 = 0
    for s, (p, n) in enumerate(zip(probs, segs)):
        W = torch.from_numpy(p.w_store.view(np.int16)).cuda().view(torch.bfloat16)
        bl.bitlinear_pack_weights(W, layout, packed=packed[r0:r0 + n], gamma=gammas[s:s + 1])
        r0 += n
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    xq, scale = bl.bitlinear_quant_acts(xt)
    y, acc = bl.bitlinear_forward_segmented(xq, scale, packed, gammas, segs, K, layout,
                                            torch.float32, acc=True)
    torch.cuda.synchronize()
    cols = 0
    for s, (p, n) in enumerate(zip(probs, segs)):
        ref = oracle.forward(p.w, probs[0].x, layout)
        assert to_np(gammas)[s] == ref["gamma"]
        codes, bad = oracle.unpack(to_np(packed)[cols:cols + n], K, layout)
        assert bad == 0
        assert check_codes(codes, ref["codes"], ref["wflags"], "codes") == 0
        assert np.array_equal(to_np(acc)[:, cols:cols + n], ref["acc"])
        check_y_f32(to_np(y)[:, cols:cols + n], ref["y64"])
        cols += n
