"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the BitLinear arithmetic: it only draws random
numbers and casts them to the storage dtype. Both the GPU path and the oracle
receive the arrays built here.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per problem, drawn in this
order): latent weights W ~ N(0, std^2) as float32 [N, K]; activations
x ~ N(0, 1) as float32 [M, K]; then, when asked for, outlier positions (exactly
round(frac * K) per token, uniform without replacement) and their signs
(+/- with p = 1/2), whose values are replaced by +/- ``outlier_value``; then the
upstream gradient for the training step. bf16 inputs are the float32 draws
cast with round-to-nearest-even (torch on the CPU); the oracle receives their
exact float32 widening.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exactly equal float32 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Problem:
    """One synthetic BitLinear problem. ``w``/``x``/``grad_y`` are the float32
    values the oracle sees (already bf16-rounded when dtype is bf16);
    ``w_store``/``x_store``/``grad_y_store`` are what the GPU receives
    (float32 arrays, or uint16 bf16 bit patterns)."""
    name: str
    M: int
    N: int
    K: int
    dtype: str
    w: np.ndarray
    x: np.ndarray
    w_store: np.ndarray
    x_store: np.ndarray
    grad_y: np.ndarray | None = None
    grad_y_store: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def make_problem(M: int, N: int, K: int, seed: int, dtype: str = "f32",
                 w_std: float = 0.02, outlier_frac: float = 0.0,
                 outlier_value: float = 20.0, grad_std: float | None = None,
                 name: str = "custom") -> Problem:
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.normal(0.0, w_std, size=(N, K)).astype(np.float32)
    x = rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out > 0:
        for m in range(M):
            pos = rng.choice(K, size=n_out, replace=False)
            sign = np.where(rng.random(n_out) < 0.5, -1.0, 1.0).astype(np.float32)
            x[m, pos] = sign * np.float32(outlier_value)
    g = None
    if grad_std is not None:
        g = rng.normal(0.0, grad_std, size=(M, N)).astype(np.float32)
    if dtype == "bf16":
        wb, xb = bf16_bits(w), bf16_bits(x)
        w, x = widen_bf16(wb), widen_bf16(xb)
        gb = None
        if g is not None:
            gb = bf16_bits(g)
            g = widen_bf16(gb)
        return Problem(name, M, N, K, dtype, w, x, wb, xb, g, gb)
    if dtype != "f32":
        raise ValueError(dtype)
    return Problem(name, M, N, K, dtype, w, x, w, x, g, g)


# Workloads: a tiny single layer, the decode GEMV, the prefill GEMM, one
# transformer block's six linear layers and the training step, with LLM-like
# shapes (hidden 4096, FFN 11008); seeds are fixed per workload.
WORKLOADS = {
    # single BitLinear forward, fp32 in and out, 2-bit packing
    "tiny": dict(M=8, N=256, K=256, seed=1, dtype="f32"),
    # decode GEMV, one token, 4096x4096, 1% outliers at +/-20
    "decode": dict(M=1, N=4096, K=4096, seed=2, dtype="bf16", outlier_frac=0.01),
    # prefill GEMM, FFN up-projection shape
    "prefill": dict(M=2048, N=11008, K=4096, seed=3, dtype="bf16"),
    # training step
    "train": dict(M=4096, N=4096, K=4096, seed=5, dtype="bf16", grad_std=1e-3),
}

# One transformer block's linear layers (hidden 4096, FFN 11008): name, N, K.
BLOCK_LAYERS = [
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("up", 11008, 4096), ("down", 4096, 11008),
]
BLOCK_SEED0 = 40


def workload(name: str, **overrides) -> Problem:
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    return make_problem(name=name, **cfg)


def block_layer(idx: int, M: int, dtype: str = "bf16") -> Problem:
    lname, N, K = BLOCK_LAYERS[idx]
    return make_problem(M=M, N=N, K=K, seed=BLOCK_SEED0 + idx, dtype=dtype, name=f"block_{lname}")
