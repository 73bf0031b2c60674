"""The allocation-free pack (bitlinear_pack_weights_noalloc) against the
workspace pack (bitlinear_pack_weights) through the C ABI: packed bytes and
the weight scale must be bit-identical, on calls in a row whose second input
is smaller (the library's scratch keeps the first call's partial sums, which
the second call must not read), over every layout and scheme."""
import numpy as np
import pytest
import torch

from ternary_weight_linear_bitlinear_amd import synth
from parity_util import guarded, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bl():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from ternary_weight_linear_bitlinear_amd import bitlinear
    return bitlinear


def dev(a, bf16):
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("layout,scheme", [("2bit", "ternary"), ("base3", "ternary"),
                                           ("2bit", "binary"), ("1bit", "binary")])
def test_noalloc_pack_matches_workspace_pack(bl, layout, scheme):
    # large first (1024 partial sums), then smaller inputs (fewer partials)
    shapes = [(4096, 4096, "bf16", 1), (300, 701, "f32", 2), (5, 17, "bf16", 3)]
    for N, K, dtype, seed in shapes:
        print(f"[case] noalloc pack {layout} {scheme} N={N} K={K} {dtype}", flush=True)
        p = synth.make_problem(M=1, N=N, K=K, seed=600 + seed, dtype=dtype)
        W = dev(p.w_store, dtype == "bf16")
        ref_packed, ref_gamma = bl.bitlinear_pack_weights(W, layout, scheme)
        rb = bl.bitlinear_packed_row_bytes(K, layout)
        packed, gp = guarded((N, rb), torch.uint8)
        gamma, gg = guarded((1,), torch.float32)
        bl.bitlinear_pack_weights_noalloc(W, packed, gamma, layout, scheme)
        torch.cuda.synchronize()
        gp.check("packed", all_written=False)
        gg.check("gamma")
        assert to_np(gamma)[0] == to_np(ref_gamma)[0], (to_np(gamma), to_np(ref_gamma))
        assert np.array_equal(to_np(packed), to_np(ref_packed)), "packed bytes differ"


def test_noalloc_pack_repeated_calls_same_result(bl):
    """Two calls in a row on the same input give the same bytes and scale."""
    p = synth.make_problem(M=1, N=64, K=4096, seed=9, dtype="bf16")
    W = dev(p.w_store, True)
    out = []
    for _ in range(2):
        packed = torch.empty((64, bl.bitlinear_packed_row_bytes(4096, "2bit")), dtype=torch.uint8,
                             device="cuda")
        gamma = torch.empty(4, dtype=torch.float32, device="cuda")[:1]
        bl.bitlinear_pack_weights_noalloc(W, packed, gamma)
        out.append((to_np(packed), to_np(gamma)))
    assert np.array_equal(out[0][0], out[1][0]) and out[0][1][0] == out[1][1][0]
