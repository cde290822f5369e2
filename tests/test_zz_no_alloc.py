"""skinny_gemm_bf16_noalloc through the C ABI: the same chooser, kernels and
bits as skinny_gemm_bf16, with the split-K partials in the library's static
scratch array (for callers that cannot allocate).  Two calls in a row, the
second smaller, each compared bit for bit with skinny_gemm_bf16 at the same
arguments and with the oracle's tolerance; a launch whose partials exceed the
array is refused before anything runs."""
import sys

import numpy as np
import pytest

import oracle
import synthetic
from tests.helpers import assert_gemm_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_FLOATS = 1 << 18


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _pair(sk, M, N, K, splits, seed):
    import torch

    x_bits, w_bits = synthetic.gemm_inputs(N=N, K=K, seed=seed)
    x, w = to_dev(x_bits[:M]), to_dev(w_bits)
    launch = sk.skinny_choose(M, N, K, splits)
    _say(f"noalloc M={M} N={N} K={K} splits={splits} launch={tuple(launch)}")
    assert launch.splits * M * N <= SCRATCH_FLOATS
    y_ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    sk.skinny_gemm_bf16(x, w, y_ref, splits)
    sk.skinny_gemm_bf16_noalloc(x, w, y_na, splits)
    torch.cuda.synchronize()
    got, want = from_dev(y_na), from_dev(y_ref)
    assert np.array_equal(got, want), f"{int(np.count_nonzero(got != want))} of {got.size} differ"
    assert_gemm_close(got, oracle.gemm_bf16(x_bits[:M], w_bits, 8), f"M={M} N={N} K={K}")
    return launch


@pytest.mark.parametrize("first,second", [
    # MFMA split-K at the largest size the array takes, then a smaller DOT2 call
    ((16, 4096, 1024, 4, 1), (5, 512, 2048, 2, 2)),
    # DOT2 split-K at the largest size, then more splits over fewer partials
    ((16, 2048, 2048, 8, 3), (1, 1024, 4096, 16, 4)),
    # the chooser's own launches (no split: the kernel or its walk)
    ((16, 1024, 4096, 0, 5), (3, 8192, 1024, 0, 6)),
    # 4 splits asked for: the chooser's 16-block launch sums them inside the
    # kernel (partials and hand-off counters in the static array), then a
    # smaller one with 2 splits
    ((16, 512, 8192, 4, 7), (9, 512, 4096, 2, 8)),    # calls the chooser runs as walks (the ring kernel, no scratch): the full
    # pooler's DOT2 walk, then a smaller off-table DOT2 walk
    ((8, 4096, 8192, 0, 9), (4, 2048, 4096, 0, 10)),
])
def test_noalloc_matches_the_allocating_call_twice(gpu_lib, first, second):
    l1 = _pair(gpu_lib, *first)
    l2 = _pair(gpu_lib, *second)
    if first[3]:
        assert l1.splits == first[3] and l2.splits == second[3]
        assert first[3] * first[0] * first[1] > second[3] * second[0] * second[1]
    if first[4] == 7:
        assert l1.path == gpu_lib.SKINNY_PATH_MFMA_4X4 and l1.splits == 4
        assert l2.path == gpu_lib.SKINNY_PATH_MFMA_4X4 and l2.splits == 2
    if first[4] == 9:
        for M, N, K, splits, _ in (first, second):
            assert gpu_lib.skinny_choose_walk(M, N, K, splits).segment > 0, (M, N, K)


def test_noalloc_refuses_partials_beyond_the_array(gpu_lib):
    import torch

    M, N, K = 16, 8192, 1024
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="static scratch"):
        gpu_lib.skinny_gemm_bf16_noalloc(x, w, y, 4)
    torch.cuda.synchronize()
    assert not y.any()
