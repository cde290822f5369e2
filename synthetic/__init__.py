"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers and rounds them to the input dtype (bfloat16, via torch's own
float32 -> bfloat16 conversion).  Both the oracle and the GPU library are fed
from here; neither imports the other.

Recipe (the decode shapes of the three API pages; no dataset, no trained
weights):
  * ``numpy.random.default_rng(seed)``; x is drawn first as float32 N(0, 1)
    for 16 rows (the largest M), then W as N(0, 1) scaled by ``w_std``
    (1/sqrt(K) by default, so y ~ N(0, 1)), then the norm weight as
    N(0, 1) * sqrt(0.1) (variance 0.1).  A call with M < 16 takes x[:M], so an
    M sweep shares W.
  * Weight rings (a distinct W per call, larger than the 256 MiB Infinity
    Cache) are drawn on the device with a seeded ``torch.Generator``,
    layer l seeded 1000 + l.
"""
from __future__ import annotations

import math

import numpy as np

MAX_M = 16


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def gemm_inputs(N: int, K: int, seed: int = 0, w_std: float | None = None,
                x_rows: int = MAX_M):
    """x bits [x_rows, K] ~ N(0,1) and W bits [N, K] ~ N(0, w_std^2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((x_rows, K), dtype=np.float32)
    std = (1.0 / math.sqrt(K)) if w_std is None else w_std
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(x), to_bf16_bits(w)


def norm_weight(P: int, seed: int = 0) -> np.ndarray:
    """Norm weight bits [P] ~ N(0, 0.1) (variance 0.1)."""
    rng = np.random.default_rng(seed + 7919)
    w = rng.standard_normal(P, dtype=np.float32) * np.float32(math.sqrt(0.1))
    return to_bf16_bits(w)


def rows_normal(M: int, P: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """bfloat16 bits [M, P] ~ N(0, std^2): rows for the norm kernels alone."""
    rng = np.random.default_rng(seed + 104729)
    r = rng.standard_normal((M, P), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(r)


def exact_integer_inputs(M: int, N: int, K: int, seed: int = 0, nnz: int = 64):
    """Integer-valued inputs whose GEMM is exact in any summation order.

    x is dense with entries in {-2..2}; each W row has at most ``nnz`` entries
    in {-2..2}, the rest zero.  Then every partial sum is an integer of
    magnitude <= 4 * nnz <= 256, exactly representable in FP32 and in
    bfloat16, so any correct implementation returns the same bits."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    w = np.zeros((N, K), dtype=np.float32)
    nnz = min(nnz, K)
    for n in range(N):
        cols = rng.choice(K, size=nnz, replace=False)
        w[n, cols] = rng.integers(-2, 3, size=nnz)
    return to_bf16_bits(x), to_bf16_bits(w)


def to_device(bits: np.ndarray, device="cuda"):
    """bfloat16 bit patterns (uint16) -> a torch bfloat16 tensor on device."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def device_weight_ring(layers: int, N: int, K: int, device, w_std: float | None = None,
                       base_seed: int = 1000):
    """``layers`` distinct W [N, K] bfloat16 tensors on ``device``, layer l
    drawn from a torch.Generator seeded base_seed + l."""
    import torch

    std = (1.0 / math.sqrt(K)) if w_std is None else w_std
    ring = []
    for l in range(layers):
        g = torch.Generator(device=device)
        g.manual_seed(base_seed + l)
        w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
        ring.append((w * std).to(torch.bfloat16))
        del w
    return ring
