"""Comparison helpers for GPU-vs-oracle parity tests.

Rules: weight codes, activation codes and INT32 accumulators are bit-exact,
except at elements the oracle flags as lying within 1e-6 relative of a
rounding boundary, which are excluded and counted; gamma and the activation
scales agree within 1e-6 relative; fp32 outputs within 1e-5 relative; bf16
outputs equal the round-to-nearest-even of the oracle's value, except where
that value is within 1e-5 relative of a bf16 rounding midpoint (then either
neighbour is accepted, and the element is counted).
"""
import numpy as np

import oracle

Y_RTOL = 1e-5
SCALE_RTOL = 1e-6


def to_np(t):
    return t.detach().cpu().numpy()


def check_codes(got_codes: np.ndarray, ref_codes: np.ndarray, flags: np.ndarray, what: str) -> int:
    bad = got_codes != ref_codes
    unflagged = bad & (flags == 0)
    assert not unflagged.any(), (
        f"{what}: {int(unflagged.sum())} unflagged mismatches, first at "
        f"{np.argwhere(unflagged)[:5].tolist()}")
    return int(bad.sum())


def check_rel(got, ref, rtol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    lim = rtol * np.abs(ref)
    badm = err > lim
    assert not badm.any(), (f"{what}: {int(badm.sum())} elements beyond rtol {rtol}; worst rel "
                            f"{float(np.max(err / np.maximum(np.abs(ref), 1e-300)))}")


def check_y_f32(y: np.ndarray, y64: np.ndarray, what="y"):
    zero = y64 == 0
    assert np.all(y[zero] == 0), f"{what}: zero accumulators must give exactly 0"
    check_rel(y[~zero], y64[~zero], Y_RTOL, what)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_y_bf16(y_bits: np.ndarray, y64: np.ndarray, what="y_bf16") -> int:
    """y_bits: uint16 bf16 patterns. Returns the number of midpoint-excluded elements."""
    ref_bits = oracle.bf16_rne(y64.astype(np.float32))
    neq = y_bits != ref_bits
    if not neq.any():
        return 0
    # distance of the exact value to the nearest bf16 midpoint
    ref = bf16_to_f64(ref_bits)
    got = bf16_to_f64(y_bits)
    lo = np.minimum(ref, got)
    hi = np.maximum(ref, got)
    mid = (lo + hi) / 2
    near_mid = np.abs(y64 - mid) <= Y_RTOL * np.abs(y64)
    # the two values must be adjacent bf16 numbers around a midpoint
    adjacent = np.abs(y_bits.astype(np.int32) - ref_bits.astype(np.int32)) == 1
    ok = near_mid & adjacent
    assert np.all(ok[neq]), f"{what}: {int((neq & ~ok).sum())} bf16 outputs differ beyond the rule"
    return int(neq.sum())


def excluded_acc_mask(xq_bad: np.ndarray, code_bad: np.ndarray) -> np.ndarray:
    """Outputs touched by a flagged (and mismatching) activation or weight code:
    rows m with any xq mismatch, columns n with any code mismatch."""
    rows = xq_bad.any(axis=1)
    cols = code_bad.any(axis=1)
    return rows[:, None] | cols[None, :]


# ----------------------------------------------------------------------------
# Canaries: outputs allocated inside a larger buffer whose bytes before and
# after the output (and the output itself, before the call) hold a fixed
# pattern. After the call the guard bytes must be intact (no write past either
# end of the output) and no output element may still hold the pattern (every
# element written: no real output equals it, since |acc| <= 127 K, codes are
# small, and y = acc * gamma * s / 127 is 0 or far above 1e-16 in magnitude
# for the test inputs).
CANARY = 0xA5
GUARD_BYTES = 4096


class Guarded:
    def __init__(self, shape, dtype, device="cuda"):
        import torch
        self.shape = tuple(int(v) for v in shape)
        self.dtype = dtype
        n = 1
        for v in self.shape:
            n *= v
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((2 * GUARD_BYTES + max(self.nbytes, 16),), CANARY,
                              dtype=torch.uint8, device=device)
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(self.shape)

    def check(self, what="output", all_written=True):
        b = to_np(self.buf)
        head, tail = b[:GUARD_BYTES], b[GUARD_BYTES + self.nbytes:]
        assert np.all(head == CANARY), f"{what}: {int((head != CANARY).sum())} bytes written before"
        assert np.all(tail == CANARY), f"{what}: {int((tail != CANARY).sum())} bytes written after"
        if all_written and self.nbytes:
            body = b[GUARD_BYTES:GUARD_BYTES + self.nbytes]
            esz = self.nbytes // max(1, int(np.prod(self.shape)))
            words = body.reshape(-1, esz)
            untouched = np.all(words == CANARY, axis=1)
            assert not untouched.any(), (f"{what}: {int(untouched.sum())} elements never written, "
                                         f"first at flat index {int(np.argmax(untouched))}")


def guarded(shape, dtype):
    """(tensor, guard) pair: pass the tensor as the output, then guard.check()."""
    g = Guarded(shape, dtype)
    return g.t, g
