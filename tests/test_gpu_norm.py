"""GPU parity of the norm kernels against the oracle, through the C ABI.

skinny_rmsnorm_nvfp4 (pooler_gather page, module description;
cvt_e2m1x8_f32, cvt_f32_to_e4m3, nvfp4_compute_output_scale): the kernel
computes in binary64 with one rounding per narrowing, as the oracle does, so
codes and scales must be bit-exact on every case (no boundary exemption).
The cases include rows built to land exactly on every e2m1 midpoint and every
e4m3 midpoint (tests/norm_cases.py), blocks whose scales are e4m3
subnormals, zero-scale blocks and signed zeros.  The boundary-exemption
rule of tests/helpers.py only explains a failure (which codes differ, and
whether they sit on a rounding boundary); it no longer accepts one.
skinny_rmsnorm_bf16 (same page, "BF16 edge layers"): bit-exact.

The full-pooler case feeds the GPU GEMM output (M=8, x[8, 8192] @ W[4096,
8192]^T) to both sides, with global_scale = 448 * 6 / amax(yn_oracle).
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synthetic
from tests import norm_cases
from tests.helpers import compare_nvfp4, from_dev, to_dev

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


def _assert_exact(r_bits, w_bits, gc, eps, gs, a, sf, tag=""):
    """Codes and scales equal to the oracle's, byte for byte.  On a mismatch
    the boundary rule names the first difference and whether it lies on a
    rounding boundary."""
    ref = oracle.rmsnorm_nvfp4(r_bits, w_bits, gc, eps, gs)
    if np.array_equal(a, ref["a"]) and np.array_equal(sf, ref["a_sf"]):
        return ref
    n_a = int(np.count_nonzero(a != ref["a"]))
    n_sf = int(np.count_nonzero(sf != ref["a_sf"]))
    try:
        exempt, total = compare_nvfp4(r_bits, w_bits, gc, eps, gs, a, sf)
        why = f"all {exempt} differing codes of {total} on a rounding boundary"
    except AssertionError as e:
        why = str(e)
    raise AssertionError(f"{tag}: {n_a} code bytes and {n_sf} scales differ; {why}")


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
    _assert_exact(r_bits, nw, gc, eps, gs, a, sf, "full pooler")
    # the block with the largest |yn| reaches the largest scale
    assert (sf == 0x7E).any()


@pytest.mark.parametrize("M,P,gc,eps", [(1, 16, 1.0, 1e-6), (3, 48, 0.0, 1e-5),
                                        (8, 4096, 1.0, 1e-6), (5, 4112, 1.0, 1e-6),
                                        (2, 8192, 0.5, 1e-2), (16, 1024, 1.0, 0.0)])
def test_nvfp4_shapes(gpu_lib, M, P, gc, eps):
    _say(f"nvfp4 M={M} P={P}")
    r = synthetic.rows_normal(M, P, seed=M * 7 + P)
    nw = synthetic.norm_weight(P, seed=P)
    for gs in (_gs_for(r, nw, gc, eps), 1.0, 3.0e4, 1.0e-3):
        a, sf = _nvfp4_gpu(gpu_lib, r, nw, gc, eps, gs)
        _assert_exact(r, nw, gc, eps, gs, a, sf, f"M={M} P={P} gs={gs}")


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
    _assert_exact(r_bits, nw, 1.0, 1e-6, 500.0, a, sf, "zero and tiny rows")


def test_nvfp4_e2m1_midpoints(gpu_lib):
    """Normed values exactly on every e2m1 midpoint {0.25, 0.75, 1.25, 1.75,
    2.5, 3.5, 5} of both signs (ties to the even code), one bfloat16 step on
    either side of each, output scales 1 and 2, saturation above 6, signed
    zeros and negative values that round to code 0x8, zero-scale blocks."""
    r, w, gc, eps, gs = norm_cases.e2m1_tie_case()
    _say(f"e2m1 ties P={w.size}")
    a, sf = _nvfp4_gpu(gpu_lib, r, w, gc, eps, gs)
    _assert_exact(r, w, gc, eps, gs, a, sf, "e2m1 midpoints")


def test_nvfp4_e4m3_midpoints(gpu_lib):
    """Block scales exactly on every e4m3fn midpoint, subnormal ones
    included (ties to the even code), on every finite e4m3fn value, and past
    448 (saturation to 0x7E)."""
    r, w, gc, eps, gs = norm_cases.e4m3_tie_case()
    _say(f"e4m3 ties P={w.size}")
    a, sf = _nvfp4_gpu(gpu_lib, r, w, gc, eps, gs)
    _assert_exact(r, w, gc, eps, gs, a, sf, "e4m3 midpoints")
    assert sorted(set(sf[0].tolist())) == list(range(0x7F))


@pytest.mark.parametrize("target", [2.0 ** -6, 2.0 ** -8])
def test_nvfp4_subnormal_scales(gpu_lib, target):
    """Normal rows with a global scale small enough that the block scales
    are e4m3 subnormals (codes 0x01..0x07) and zero, the largest block at or
    near the smallest normal 0x08."""
    r, w, gc, eps, gs_of = norm_cases.subnormal_scale_case(gs_target=target)
    gs = gs_of(oracle.bf16_value(oracle.rmsnorm_bf16(r, w, gc, eps)))
    _say(f"subnormal scales target={target} gs={gs}")
    a, sf = _nvfp4_gpu(gpu_lib, r, w, gc, eps, gs)
    _assert_exact(r, w, gc, eps, gs, a, sf, f"subnormal scales {target}")
    assert np.count_nonzero((sf >= 1) & (sf <= 7)) > 0.5 * sf.size


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
    ref_bits = oracle.rmsnorm_bf16(r_bits, nw, 1.0, 1e-6)
    y = torch.empty((M, P), dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_rmsnorm_bf16(to_dev(r_bits), to_dev(nw), 1.0, 1e-6, y)
    torch.cuda.synchronize()
    got = from_dev(y)
    bad = int(np.count_nonzero(got != ref_bits))
    assert bad == 0, f"{bad} of {ref_bits.size} differ"


def test_rmsnorm_bf16_signed_zeros_and_exact_rows(gpu_lib):
    """The constructed +-1 rows (normed value exactly r * (w + 0)), with
    -0.0 and +0.0 weights: bit for bit, signs of zero included."""
    import torch

    r_bits, nw, gc, eps, _ = norm_cases.e2m1_tie_case()
    ref_bits = oracle.rmsnorm_bf16(r_bits, nw, gc, eps)
    y = torch.empty(r_bits.shape, dtype=torch.bfloat16, device="cuda")
    gpu_lib.skinny_rmsnorm_bf16(to_dev(r_bits), to_dev(nw), gc, eps, y)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(y), ref_bits)


def test_norm_deterministic(gpu_lib):
    r_bits = synthetic.rows_normal(8, 4096, seed=3)
    nw = synthetic.norm_weight(4096, seed=3)
    first = _nvfp4_gpu(gpu_lib, r_bits, nw, 1.0, 1e-6, 100.0)
    for _ in range(5):
        again = _nvfp4_gpu(gpu_lib, r_bits, nw, 1.0, 1e-6, 100.0)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
