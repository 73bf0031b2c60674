"""Pins for the CPU oracle: every expected value here comes from the pages'
printed numbers, exact rational arithmetic, brute force, closed forms or a
library routine, never from the oracle itself.

Pages (cited by title and section):
  [b158]   BitNet b1.58深度解析：三值权重如何重塑大模型推理
  [QAT-en] QAT and BitNet: A Deep Dive into 1-bit and 1.58-bit
           Quantization-Aware Training
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_bitlinear_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def f32(v):
    return np.asarray(v, dtype=np.float32)


def frac_to_f32_rne(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    cand = np.float32(float(fr))
    best = None
    for c in (np.nextafter(cand, np.float32(-np.inf)), cand, np.nextafter(cand, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


# ----------------------------------------------------------------------------
# Worked examples printed on the pages
def test_absmean_worked_example(golden):
    """[b158] §3.1 example: gamma 0.61, W_norm and codes as printed."""
    ex = golden["absmean_example"]
    W = f32(ex["W"])[None, :]
    codes, flags, gamma = oracle.ternary_codes(W)
    assert round(float(gamma), 2) == ex["gamma_printed"]
    w_norm = W[0].astype(np.float64) / (float(gamma) + 1e-5)
    assert [round(v, 2) for v in w_norm.tolist()] == ex["W_norm_printed"]
    assert codes[0].tolist() == ex["codes_printed"]
    assert flags.sum() == 0


def test_five_weight_example(golden):
    """[QAT-en] 'A Five-Weight Example': ternary gamma 0.57 zeroes 0.05 (error
    0.05); 1-bit beta 0.57 pushes it to +0.57 (error 0.52); the other four
    weights are the same in both versions."""
    ex = golden["five_weight_example"]
    w = f32(ex["w"])[None, :]
    i = ex["index_of_small_weight"]
    tc, tflags, gamma = oracle.ternary_codes(w)
    bc, bflags, alpha, beta = oracle.binary_codes(w)
    assert round(float(gamma), 2) == ex["gamma_printed"]
    assert round(float(beta), 2) == ex["beta_printed"]
    t_val = float(gamma) * tc[0, i]
    b_val = float(beta) * bc[0, i]
    assert t_val == ex["ternary_value_of_small_weight"]
    assert round(abs(t_val - float(w[0, i])), 2) == ex["ternary_error_printed"]
    assert round(b_val, 2) == ex["binary_value_of_small_weight"]
    assert round(abs(b_val - float(w[0, i])), 2) == ex["binary_error_printed"]
    others = [j for j in range(w.shape[1]) if j != i]
    assert np.array_equal(tc[0, others], bc[0, others])
    assert set(tc[0].tolist()) <= {-1, 0, 1} and set(bc[0].tolist()) <= {-1, 1}
    assert tflags.sum() == 0 and bflags.sum() == 0


# ----------------------------------------------------------------------------
# gamma and alpha against exact rational arithmetic
@pytest.mark.parametrize("shape,seed", [((1, 5), 0), ((3, 7), 1), ((17, 33), 2), ((64, 80), 3)])
def test_absmean_exact(shape, seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, size=shape).astype(np.float32)
    w[0, 0] = np.float32(3.0)  # spread the exponents
    exact = sum(Fraction(float(v)) for v in np.abs(w).ravel()) / w.size
    g32, g64 = oracle.absmean(w)
    assert g32 == frac_to_f32_rne(exact)
    assert abs(Fraction(g64) - exact) <= exact * Fraction(1, 10**14)
    m32, _ = oracle.mean(w)
    exact_m = sum(Fraction(float(v)) for v in w.ravel()) / w.size
    assert m32 == frac_to_f32_rne(exact_m)


# ----------------------------------------------------------------------------
# 1-bit codes: centred by the mean alpha, not by zero
def test_binary_codes_hand_example():
    """[QAT-en] 'The BitLinear Recipe', step 2: alpha is the mean of the
    weights; weights above it become +1, weights below it -1; step 4 rescales
    by beta = mean|W|. Worked by hand: w = [1, 2, 3, 4, 5] has alpha = 3 and
    beta = 3, so the codes are [-1, -1, -1, +1, +1] (the weight equal to alpha
    takes -1, the reading for a tie). Centring on zero instead of alpha would
    give five +1 codes."""
    w = f32([[1.0, 2.0, 3.0, 4.0, 5.0]])
    codes, flags, alpha, beta = oracle.binary_codes(w)
    assert alpha == np.float32(3.0) and beta == np.float32(3.0)
    assert codes[0].tolist() == [-1, -1, -1, 1, 1]
    assert flags[0].tolist() == [0, 0, 1, 0, 0]  # only the tie is flagged
    # negative weights: alpha = -2, codes of -1 and 0 are +1 although -1 < 0
    w = f32([[-5.0, -3.0, -1.0, 0.0, -1.0]])
    codes, _, alpha, beta = oracle.binary_codes(w)
    assert alpha == np.float32(-2.0) and beta == np.float32(2.0)
    assert codes[0].tolist() == [-1, -1, 1, 1, 1]


@pytest.mark.parametrize("seed,mu", [(0, 0.05), (1, -0.03)])
def test_binary_codes_exact_centring(seed, mu):
    """On a matrix whose mean is far from zero, every unflagged code is the
    sign of w - alpha against the exact rational mean (many weights lie
    between 0 and alpha, so a sign test around 0 fails here)."""
    rng = np.random.default_rng(seed)
    w = rng.normal(mu, 0.02, size=(12, 50)).astype(np.float32)
    codes, flags, alpha, beta = oracle.binary_codes(w)
    exact = sum(Fraction(float(v)) for v in w.ravel()) / w.size
    ref = np.array([1 if Fraction(float(v)) > exact else -1 for v in w.ravel()],
                   np.int8).reshape(w.shape)
    between = ((w > 0) & (w.astype(np.float64) < float(exact))) | \
              ((w < 0) & (w.astype(np.float64) > float(exact)))
    assert between.sum() > 50  # the case discriminates centring
    ok = flags == 0
    assert ok.sum() >= w.size - 2
    assert np.array_equal(codes[ok], ref[ok])
    exact_abs = sum(Fraction(float(v)) for v in np.abs(w).ravel()) / w.size
    assert beta == frac_to_f32_rne(exact_abs)


# ----------------------------------------------------------------------------
# Ternary codes: the threshold form and the code set
def _threshold_codes_exact(w: np.ndarray, d: np.float32):
    """[QAT-en] 'The Ternary Weight Recipe', equivalent form: |w| <= d/2 -> 0,
    w > d/2 -> +1, w < -d/2 -> -1, evaluated in exact rationals."""
    half = Fraction(float(d)) / 2
    out = []
    for v in w.ravel():
        fv = Fraction(float(v))
        out.append(0 if abs(fv) <= half else (1 if fv > 0 else -1))
    return np.array(out, np.int8).reshape(w.shape)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_threshold_form(seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, size=(24, 40)).astype(np.float32)
    codes, flags, gamma = oracle.ternary_codes(w)
    d = np.float32(gamma + np.float32(1e-5))
    # plant weights on and next to the boundary d/2 (an exact float32 value)
    half = np.float32(d / np.float32(2))
    w[0, :6] = [half, -half, np.nextafter(half, np.float32(1)), -np.nextafter(half, np.float32(1)),
                np.nextafter(half, np.float32(0)), 3 * d]
    codes, flags, _ = oracle.ternary_codes(w, gamma=gamma)
    ref = _threshold_codes_exact(w, d)
    ok = flags == 0
    assert np.array_equal(codes[ok], ref[ok])
    # exactly on the boundary: the quotient is 0.5, half to even gives 0
    assert codes[0, 0] == 0 and codes[0, 1] == 0
    assert codes[0, 5] == 1
    assert flags[0, :5].all()


def test_code_set_and_clamp():
    w = f32([[0.0, 1e30, -1e30, 1e-30, -0.0, 5.0, -5.0, 0.01]])
    codes, _, _ = oracle.ternary_codes(w)
    assert set(np.unique(codes).tolist()) <= {-1, 0, 1}
    assert codes[0].tolist()[:3] == [0, 1, -1]


def test_gaussian_zero_fraction():
    """Closed form: for W ~ N(0, s^2) the absmean is s*sqrt(2/pi), and a code
    is 0 iff |w| <= (gamma + eps)/2, so P(0) = erf((gamma+eps)/(2 s sqrt 2))
    = erf(1/(2 sqrt(pi))) = 0.3101 when eps -> 0; +1 and -1 split the rest."""
    s = 0.02
    p = synth.make_problem(M=1, N=2048, K=2048, seed=11)
    codes, _, gamma = oracle.ternary_codes(p.w)
    g = s * math.sqrt(2 / math.pi)
    p0 = math.erf((g + 1e-5) / (2 * s * math.sqrt(2)))
    assert abs(math.erf(1 / (2 * math.sqrt(math.pi))) - 0.3101) < 1e-4
    n = codes.size
    sd = math.sqrt(p0 * (1 - p0) / n)
    assert abs((codes == 0).mean() - p0) < 5 * sd + 1e-4
    sdp = math.sqrt(0.5 * (1 - p0) * (1 - 0.5 * (1 - p0)) / n)
    assert abs((codes == 1).mean() - (1 - p0) / 2) < 5 * sdp + 1e-4
    assert abs(float(gamma) - g) / g < 5e-3


# ----------------------------------------------------------------------------
# Packing
def test_pack_2bit_hand_example():
    """One 16-code group, bytes worked out by hand from the layout: byte i of
    the group holds codes i, 4+i, 8+i, 12+i (2 bits each, low bits first),
    stored as u = c + 1; the rest of the 16-byte row is padding u = 1 (0x55)."""
    c = np.array([[-1, 0, 1, 1, 0, 0, -1, 1, 1, 1, 1, 1, -1, -1, -1, 0]], np.int8)
    packed = oracle.pack(c, "2bit")
    assert packed.shape == (1, 16)
    assert packed[0].tolist() == [0x24, 0x25, 0x22, 0x6A] + [0x55] * 12


def test_pack_2bit_word_extraction():
    """The layout's decode law: for each little-endian 32-bit word (16 codes),
    (word >> 2j) & 0x03030303 holds u = c + 1 of codes 4j..4j+3 in its bytes."""
    rng = np.random.default_rng(5)
    c = rng.integers(-1, 2, size=(3, 128)).astype(np.int8)
    words = oracle.pack(c, "2bit").view("<u4")
    u = (c.astype(np.int32) + 1)
    for n in range(3):
        for g in range(8):
            for j in range(4):
                v = (int(words[n, g]) >> (2 * j)) & 0x03030303
                got = [(v >> (8 * b)) & 0xFF for b in range(4)]
                assert got == u[n, 16 * g + 4 * j:16 * g + 4 * j + 4].tolist()


def test_pack_base3_hand_example():
    """Five codes per byte as t0 + 3 t1 + 9 t2 + 27 t3 + 81 t4 with t = c + 1:
    [-1, 0, 1, 1, -1] -> 0 + 3 + 18 + 54 + 0 = 75; [1, -1] plus three pad trits
    (t = 1) -> 2 + 0 + 9 + 27 + 81 = 119; a full pad byte is 121."""
    c = np.array([[-1, 0, 1, 1, -1, 1, -1]], np.int8)
    packed = oracle.pack(c, "base3")
    assert packed.shape == (1, 16)
    assert packed[0].tolist() == [75, 119] + [121] * 14


@pytest.mark.parametrize("layout", ["2bit", "base3"])
@pytest.mark.parametrize("K", [1, 3, 4, 5, 15, 16, 17, 63, 64, 65, 79, 80, 81, 255, 4096])
def test_pack_roundtrip(layout, K):
    rng = np.random.default_rng(K)
    c = rng.integers(-1, 2, size=(5, K)).astype(np.int8)
    packed = oracle.pack(c, layout)
    back, bad = oracle.unpack(packed, K, layout)
    assert bad == 0
    assert np.array_equal(back, c)


def test_every_2bit_byte():
    """81 of the 256 byte values are valid (no field holds the pattern 11);
    each decodes and re-encodes to itself; the other 175 are reported."""
    valid = 0
    for b in range(256):
        row = np.full((1, 16), 0x55, np.uint8)
        row[0, 0] = b
        codes, bad = oracle.unpack(row, 16, "2bit")
        fields = [(b >> (2 * j)) & 3 for j in range(4)]
        if 3 in fields:
            assert bad == fields.count(3)
            continue
        valid += 1
        assert bad == 0
        assert np.array_equal(oracle.pack(codes, "2bit"), row)
        assert [codes[0, 4 * j] for j in range(4)] == [f - 1 for f in fields]
    assert valid == 3 ** 4


def test_every_base3_byte():
    """243 = 3^5 byte values are valid and round-trip; 243..255 are reported."""
    for b in range(256):
        row = np.full((1, 16), 121, np.uint8)
        row[0, 0] = b
        codes, bad = oracle.unpack(row, 5, "base3")
        if b >= 243:
            assert bad == 1
            continue
        assert bad == 0
        digits = [(b // 3 ** i) % 3 - 1 for i in range(5)]
        assert codes[0].tolist() == digits
        assert np.array_equal(oracle.pack(codes, "base3"), row)


def test_pack_1bit_hand_example():
    """One 32-code group of +-1 codes, bytes worked out by hand from the
    layout: code k sits in byte k % 4 at bit k // 4, bit 1 = +1. +1 at k = 0
    (byte 0 bit 0), 5 (byte 1 bit 1), 10 (byte 2 bit 2), 15 (byte 3 bit 3) and
    31 (byte 3 bit 7), -1 elsewhere; the rest of the 16-byte row is padding 0."""
    c = -np.ones((1, 32), np.int8)
    c[0, [0, 5, 10, 15, 31]] = 1
    packed = oracle.pack(c, "1bit")
    assert packed.shape == (1, 16)
    assert packed[0].tolist() == [0x01, 0x02, 0x04, 0x88] + [0] * 12


def test_pack_1bit_word_extraction():
    """The layout's decode law: for each little-endian 32-bit word (32 codes),
    (word >> j) & 0x01010101 holds, byte by byte, the bits of codes 4j..4j+3
    (1 for +1)."""
    rng = np.random.default_rng(6)
    c = np.where(rng.random((3, 256)) < 0.5, -1, 1).astype(np.int8)
    words = oracle.pack(c, "1bit").view("<u4")
    for n in range(3):
        for g in range(8):
            for j in range(8):
                v = (int(words[n, g]) >> j) & 0x01010101
                got = [(v >> (8 * b)) & 0xFF for b in range(4)]
                want = [1 if c[n, 32 * g + 4 * j + b] == 1 else 0 for b in range(4)]
                assert got == want


@pytest.mark.parametrize("K", [1, 7, 8, 9, 31, 32, 33, 127, 128, 129, 1000, 4096])
def test_pack_1bit_roundtrip(K):
    rng = np.random.default_rng(K + 1)
    c = np.where(rng.random((5, K)) < 0.5, -1, 1).astype(np.int8)
    packed = oracle.pack(c, "1bit")
    assert packed.shape == (5, ((K + 7) // 8 + 15) // 16 * 16)
    back, bad = oracle.unpack(packed, K, "1bit")
    assert bad == 0
    assert np.array_equal(back, c)


def test_every_1bit_byte():
    """All 256 byte values are valid; byte 0 of a row holds codes 0, 4, ..., 28."""
    for b in range(256):
        row = np.zeros((1, 16), np.uint8)
        row[0, 0] = b
        codes, bad = oracle.unpack(row, 32, "1bit")
        assert bad == 0
        assert [codes[0, 4 * j] for j in range(8)] == [1 if (b >> j) & 1 else -1
                                                       for j in range(8)]
        assert np.array_equal(oracle.pack(codes, "1bit"), row)


def test_pack_1bit_rejects_ternary_zero():
    c = np.array([[1, -1, 0, 1]], np.int8)
    with pytest.raises(ValueError):
        oracle.pack(c, "1bit")


def test_one_bit_storage(golden):
    """[QAT-en] "What Does BitLinear Change?": +-1 weights take 1 bit each,
    16x below FP16; rows of a multiple of 128 codes carry no padding."""
    ex = golden["one_bit_storage"]
    ratio = ex["bits_per_weight_fp16_printed"] / ex["bits_per_weight_1bit_printed"]
    for K in (128, 4096, 11008):
        assert 8 * oracle.row_bytes(K, "1bit") / K == ex["bits_per_weight_1bit_printed"]
        assert 2 * K / oracle.row_bytes(K, "1bit") == ratio  # FP16 bytes over 1-bit bytes


def test_binary_forward_same_in_both_containers():
    """The 1-bit codes stored in one bit or in the 2-bit container unpack to the
    same codes, so the whole forward pass agrees."""
    rng = np.random.default_rng(8)
    w = rng.normal(0, 0.02, size=(40, 300)).astype(np.float32)
    x = rng.normal(0, 1, size=(3, 300)).astype(np.float32)
    a = oracle.forward(w, x, "1bit", "binary")
    b = oracle.forward(w, x, "2bit", "binary")
    assert np.array_equal(oracle.unpack(a["packed"], 300, "1bit")[0],
                          oracle.unpack(b["packed"], 300, "2bit")[0])
    assert np.array_equal(a["acc"], b["acc"]) and np.array_equal(a["y64"], b["y64"])


def test_storage_arithmetic(golden):
    """[b158] §4.1: 70B weights take 140 GB in FP16, 17.5 GB at 2 bits and about
    14 GB at five per byte; 1.6 bits per weight, about 10x below FP16."""
    ex = golden["storage_arithmetic"]
    P = ex["params_70B"]
    K = 8000  # a row length with no padding in either layout
    N = P // K
    assert oracle.row_bytes(K, "2bit") == K // ex["weights_per_byte_2bit"]
    assert oracle.row_bytes(K, "base3") == K // ex["weights_per_byte_base3"]
    assert 2 * P == ex["fp16_bytes_printed"]
    assert N * oracle.row_bytes(K, "2bit") == ex["two_bit_bytes_printed"]
    assert N * oracle.row_bytes(K, "base3") == ex["five_per_byte_bytes_printed_approx"]
    assert 3 ** 5 == ex["base3_states"] <= 256
    assert 8 / ex["weights_per_byte_base3"] == ex["bits_per_weight_base3_printed"]
    assert round(16 / (8 / ex["weights_per_byte_base3"])) == ex["fp16_ratio_printed_approx"]


# ----------------------------------------------------------------------------
# Activation quantiser
def test_quant_acts_invariants():
    """[b158] §3.2: per-token scale = max|x|; codes in [-127, 127]; the
    largest-magnitude element maps to +/-127; dequantisation error at most
    s/254; non-boundary codes are the nearest integer to 127 x / s."""
    p = synth.make_problem(M=6, N=1, K=4096, seed=2, dtype="bf16", outlier_frac=0.01)
    x = p.x.copy()
    x[5] = 0.0  # an all-zero token
    xq, scale, flags = oracle.quant_acts(x)
    assert xq.min() >= -127 and xq.max() <= 127
    for m in range(5):
        s = np.abs(x[m]).max()
        assert scale[m] == s
        k = np.abs(x[m]).argmax()
        assert abs(int(xq[m, k])) == 127 and np.sign(xq[m, k]) == np.sign(x[m, k])
        deq = xq[m].astype(np.float64) * float(s) / 127.0
        assert np.all(np.abs(deq - x[m]) <= float(s) / 254.0 * (1 + 1e-6))
        exact = x[m].astype(np.float64) * 127.0 / float(s)
        ok = flags[m] == 0
        assert np.array_equal(xq[m][ok], np.rint(exact[ok]).astype(np.int8))
    assert scale[5] == np.float32(1e-6) and not xq[5].any()


def _planted_ties():
    """Rows whose fp32 steps x / s, then * 127 land exactly on k + 1/2 for
    k = 0..126 (found by searching the float32 neighbourhood of (k + 1/2) s /
    127; s is the row's largest |x|, planted as the first element)."""
    rows, ks = [], []
    for s in (np.float32(127.0), np.float32(20.0), np.float32(3.0)):
        row, krow = [s], [None]
        for k in range(127):
            target = np.float32(k + 0.5)
            x0 = np.float32(target * s / np.float32(127))
            for d in (0, 1, -1, 2, -2, 3, -3):
                x = x0
                for _ in range(abs(d)):
                    x = np.nextafter(x, np.float32(np.inf if d > 0 else -np.inf))
                if abs(x) <= s and np.float32(np.float32(x / s) * np.float32(127)) == target:
                    row += [x, -x]
                    krow += [k, -k - 1]  # -x lands on -(k + 1/2), between -k-1 and -k
                    break
        rows.append((np.array(row, np.float32), krow))
    return rows


def test_quant_acts_ties_round_half_to_even():
    """[b158] §3.2 and §5.2 round with torch.round, which rounds a value
    exactly halfway between two integers to the even one. Planted elements
    whose fp32 quotient times 127 is exactly k + 1/2 must give the even
    neighbour (k for even k, k + 1 for odd k; mirrored for negative values),
    not the neighbour away from zero."""
    n_even = 0
    for row, krow in _planted_ties():
        xq, scale, flags = oracle.quant_acts(row[None, :])
        assert scale[0] == row[0] and xq[0, 0] == 127
        for j in range(1, row.size):
            lo = krow[j]  # the value lies in (lo, lo + 1), exactly halfway
            expect = lo if lo % 2 == 0 else lo + 1
            assert xq[0, j] == expect, (row[0], row[j], lo, xq[0, j])
            assert flags[0, j] == 1
            n_even += (lo >= 0 and lo % 2 == 0)
    assert n_even >= 150


def test_quant_acts_outliers_hit_127():
    """With +/-20 outliers the outliers define the scale and map to +/-127."""
    p = synth.workload("decode")
    xq, scale, _ = oracle.quant_acts(p.x)
    out = np.abs(p.x[0]) == 20.0
    assert out.sum() == 41
    assert scale[0] == 20.0
    assert np.all(np.abs(xq[0][out]) == 127)


# ----------------------------------------------------------------------------
# Integer product and epilogue
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 16, 64), (17, 9, 130)])
def test_int_product_bruteforce(M, N, K):
    rng = np.random.default_rng(M * 100 + N)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    c = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    acc = oracle.int_product(xq, c)
    ref = xq.astype(np.int64) @ c.astype(np.int64).T
    assert np.array_equal(acc, ref.astype(np.int32))


def test_int_product_all_243_code_vectors():
    """Exhaustive K = 5: every ternary code vector against random INT8 rows,
    checked against add/subtract/skip written out per element ([b158] §4.2)."""
    import itertools
    c = np.array(list(itertools.product([-1, 0, 1], repeat=5)), np.int8)
    rng = np.random.default_rng(9)
    xq = rng.integers(-127, 128, size=(4, 5)).astype(np.int8)
    acc = oracle.int_product(xq, c)
    for m in range(4):
        for n in range(243):
            s = 0
            for k in range(5):
                if c[n, k] == 1:
                    s += int(xq[m, k])
                elif c[n, k] == -1:
                    s -= int(xq[m, k])
            assert acc[m, n] == s
    u = c.astype(np.int64) + 1
    assert np.array_equal(acc, xq.astype(np.int64) @ u.T - xq.astype(np.int64).sum(1, keepdims=True))


def test_int_product_overflow_detected():
    K = 2147483647 // 127 + 1
    xq = np.full((1, K), 127, np.int8)
    c = np.ones((1, K), np.int8)
    with pytest.raises(OverflowError):
        oracle.int_product(xq, c)


def test_epilogue_matches_float_form():
    """[b158] §5.2-5.3: F.linear(x_q / 127 * scale, W_q) * gamma, in fp64 with
    numpy, equals the integer product dequantised by gamma * scale / 127."""
    p = synth.workload("tiny")
    r = oracle.forward(p.w, p.x)
    xdeq = r["xq"].astype(np.float64) / 127.0 * r["scale"].astype(np.float64)[:, None]
    yf = (xdeq @ r["codes"].astype(np.float64).T) * float(r["gamma"])
    nz = r["acc"] != 0
    assert np.all(r["y64"][~nz] == 0.0)
    assert np.max(np.abs(yf[nz] - r["y64"][nz]) / np.abs(r["y64"][nz])) < 1e-12


def test_tiny_forward_close_to_unquantised():
    """Sanity: the quantised layer tracks x W^T (relative Frobenius error of a
    ternary/INT8 layer on Gaussian data is far below 1)."""
    p = synth.workload("tiny")
    r = oracle.forward(p.w, p.x)
    y = p.x.astype(np.float64) @ p.w.astype(np.float64).T
    err = np.linalg.norm(r["y64"] - y) / np.linalg.norm(y)
    assert err < 0.6


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    f = rng.normal(0, 1, 4096).astype(np.float32)
    ties = (np.arange(64, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, f32([0.0, -0.0, 1.0, 1.00390625, 1.01171875])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(f), ref)


# ----------------------------------------------------------------------------
# Training step (identity straight-through estimator)
def test_ste_grads_match_autograd():
    """[QAT-en] 'How Gradients Flow': the backward treats rounding as the
    identity. With gamma held constant, y = gamma * x Wq^T with
    Wq = W/gamma + (codes - W/gamma).detach() gives, by torch autograd in fp64,
    grad_x = grad_y (gamma codes) and grad_W = grad_y^T x."""
    p = synth.make_problem(M=12, N=10, K=24, seed=21, grad_std=1e-3)
    codes, _, gamma = oracle.ternary_codes(p.w)
    g = float(gamma)
    W = torch.tensor(p.w, dtype=torch.float64, requires_grad=True)
    x = torch.tensor(p.x, dtype=torch.float64, requires_grad=True)
    c = torch.tensor(codes, dtype=torch.float64)
    Wq = W / g + (c - W / g).detach()
    y = g * (x @ Wq.T)
    y.backward(torch.tensor(p.grad_y, dtype=torch.float64))
    gx = oracle.ste_grad_x(p.grad_y, codes, gamma)
    gw = oracle.ste_grad_w(p.grad_y, p.x)
    assert np.allclose(gx, x.grad.numpy(), rtol=1e-12, atol=1e-18)
    assert np.allclose(gw, W.grad.numpy(), rtol=1e-12, atol=1e-18)
