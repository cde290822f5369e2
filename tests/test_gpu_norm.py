"""GPU parity of the norm kernels against the oracle, through the C ABI.

skinny_rmsnorm_nvfp4 (pooler_gather page, module description): codes and
scales bit-exact except where the oracle's pre-quantization value lies within
one bfloat16 ulp (scaled) of a rounding boundary (tests/helpers.py); the
number of exempt positions must stay below 1%.
skinny_rmsnorm_bf16 (same page, "BF16 edge layers"): within one bfloat16 ulp
of the oracle, with fewer than 1% of elements off by that ulp.

The full-pooler case feeds the GPU GEMM output (M=8, x[8, 8192] @ W[4096,
8192]^T) to both sides, with global_scale = 448 * 6 / amax(yn_oracle).
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synthetic
from tests.helpers import bf16_ulp, compare_nvfp4, from_dev, to_dev

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _nvfp4_gpu(sk, r_bits, w_bits, gc, eps, gs):
    import torch

    M, P = r_bits.shape
    r = to_dev(r_bits)
    w = to_dev(w_bits)
    g = torch.tensor([oracle.f32(gs)], dtype=torch.float32, device="cuda")
    a = torch.full((M, P // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((M, P // 16), 0xCD, dtype=torch.uint8, device="cuda")
    sk.skinny_rmsnorm_nvfp4(r, w, gc, eps, g, a, sf)
    torch.cuda.synchronize()
    return a.cpu().numpy(), sf.cpu().numpy()


def _gs_for(r_bits, w_bits, gc, eps):
    yn = oracle.bf16_value(oracle.rmsnorm_bf16(r_bits, w_bits, gc, eps))
    return oracle.f32(448.0 * 6.0 / np.abs(yn).max())


def test_full_pooler_expert_input(gpu_lib):
    """GEMM -> RMSNorm -> NVFP4 at M=8, P=4096, eps 1e-6, gain center 1."""
    import torch

    M, N, K = 8, 4096, 8192
    _say("full pooler M=8 -> nvfp4")
    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=11)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_gemm_bf16(to_dev(x_bits[:M]), to_dev(w_bits), y, 0)
    torch.cuda.synchronize()
    r_bits = from_dev(y)
    nw = synthetic.norm_weight(N, seed=11)
    gc, eps = 1.0, 1e-6
    gs = _gs_for(r_bits, nw, gc, eps)
    a, sf = _nvfp4_gpu(gpu_lib, r_bits, nw, gc, eps, gs)
    exempt, total = compare_nvfp4(r_bits, nw, gc, eps, gs, a, sf)
    _say(f"exempt {exempt} of {total}")
    assert exempt < 0.01 * total
    # the block with the largest |yn| reaches the largest scale
    assert (sf == 0x7E).any()


@pytest.mark.parametrize("M,P,gc,eps", [(1, 16, 1.0, 1e-6), (3, 48, 0.0, 1e-5),
                                        (8, 4096, 1.0, 1e-6), (5, 4112, 1.0, 1e-6),
                                        (2, 8192, 0.5, 1e-2), (16, 1024, 1.0, 0.0)])
def test_nvfp4_shapes(gpu_lib, M, P, gc, eps):
    _say(f"nvfp4 M={M} P={P}")
    r = synthetic.rows_normal(M, P, seed=M * 7 + P)
    nw = synthetic.norm_weight(P, seed=P)
    for gs in (_gs_for(r, nw, gc, eps), 1.0, 3.0e4):
        a, sf = _nvfp4_gpu(gpu_lib, r, nw, gc, eps, gs)
        exempt, total = compare_nvfp4(r, nw, gc, eps, gs, a, sf)
        assert exempt <= max(2, 0.01 * total)


def test_nvfp4_zero_and_tiny_rows(gpu_lib):
    """All-zero blocks give scale 0 and code 0; a row of one repeated value
    and a row with a single non-zero exercise the closed forms."""
    P = 256
    r = np.zeros((3, P), dtype=np.float32)
    r[1, :] = 0.75
    r[2, 100] = 3.0
    r_bits = synthetic.to_bf16_bits(r)
    nw = synthetic.norm_weight(P, seed=1)
    a, sf = _nvfp4_gpu(gpu_lib, r_bits, nw, 1.0, 1e-6, 500.0)
    assert np.all(sf[0] == 0) and np.all(a[0] == 0)
    exempt, _ = compare_nvfp4(r_bits, nw, 1.0, 1e-6, 500.0, a, sf)
    assert exempt <= 2


def test_golden_worked_block_on_gpu(gpu_lib):
    """The hand-worked example of tests/golden/nvfp4_worked.txt, on the GPU."""
    r = synthetic.to_bf16_bits(np.array([[6, -4, 2, 2, 1, -1, 1, 1] + [0] * 8], dtype=np.float32))
    w = synthetic.to_bf16_bits(np.zeros(16, dtype=np.float32))
    a, sf = _nvfp4_gpu(gpu_lib, r, w, 1.0, 0.0, 896.0)
    assert list(a[0]) == [0xE7, 0x44, 0xA2, 0x22, 0, 0, 0, 0]
    assert int(sf[0, 0]) == 0x7E


@pytest.mark.parametrize("M,P", [(8, 4096), (1, 16), (5, 4112), (3, 8192)])
def test_rmsnorm_bf16(gpu_lib, M, P):
    import torch

    _say(f"rmsnorm_bf16 M={M} P={P}")
    r_bits = synthetic.rows_normal(M, P, seed=P + M)
    nw = synthetic.norm_weight(P, seed=P)
    ref = oracle.bf16_value(oracle.rmsnorm_bf16(r_bits, nw, 1.0, 1e-6))
    y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_rmsnorm_bf16(to_dev(r_bits), to_dev(nw), 1.0, 1e-6, y)
    torch.cuda.synchronize()
    got = oracle.bf16_value(from_dev(y))
    diff = np.abs(got - ref)
    assert np.all(diff <= bf16_ulp(ref))
    assert (diff > 0).sum() <= max(2, 0.01 * ref.size)


def test_norm_deterministic(gpu_lib):
    r_bits = synthetic.rows_normal(8, 4096, seed=3)
    nw = synthetic.norm_weight(4096, seed=3)
    first = _nvfp4_gpu(gpu_lib, r_bits, nw, 1.0, 1e-6, 100.0)
    for _ in range(5):
        again = _nvfp4_gpu(gpu_lib, r_bits, nw, 1.0, 1e-6, 100.0)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
