"""GPU GEMM on non-finite operands, through the C ABI.

The pages do not speak of Inf or NaN operands; the reading taken here is
IEEE arithmetic on the exact sum: an output is NaN when a NaN operand, a
0 x Inf product or both +Inf and -Inf terms enter its sum, +-Inf when Inf
terms of one sign do, and finite otherwise.  That class does not depend on
the order of the additions (with x ~ N(0, 1) and W ~ N(0, 1/K) no finite
FP32 partial sum comes near overflow), so every path, split count, walk and
ring launch must give the oracle's class at every element, and the finite
elements stay within the GEMM tolerance.

Injected values (bfloat16 bits), so that every case keeps finite outputs
too: weight row 10 takes -Inf and row 20 both +Inf and -Inf; row 30 takes
+Inf where token 0 is zero (0 x Inf: NaN for token 0, +-Inf for the others);
from 2 tokens on, token 1 takes a NaN (its whole row of y is NaN); from 3,
the last token takes -Inf at the last K (the ragged-tail loads) with a zero
weight in row 3 there; from 4, token 2 takes +Inf.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synthetic
from tests.helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)
INF, NINF, NAN = 0x7F80, 0xFF80, 0x7FC0


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(M, N, K, seed):
    x, w = synthetic.gemm_inputs(N=N, K=K, seed=seed)
    x = x[:M].copy()
    w = w.copy()
    w[10, 200] = NINF
    w[20, 300] = INF
    w[20, 301] = NINF
    x[0, 400] = 0
    w[30, 400] = INF
    if M >= 2:
        x[1, 100] = NAN
    if M >= 3:
        x[M - 1, K - 1] = NINF
        w[3, K - 1] = 0
    if M >= 4:
        x[2, 5] = INF
    return x, w


def _assert_same_class(y_gpu, y_ref, what):
    g = oracle.bf16_value(y_gpu)
    r = oracle.bf16_value(y_ref)
    for name, f in (("NaN", np.isnan), ("+Inf", np.isposinf), ("-Inf", np.isneginf)):
        diff = np.argwhere(f(g) != f(r))
        assert not len(diff), (f"{what}: {len(diff)} elements differ in being {name}; first "
                               f"{tuple(diff[0])}: gpu {g[tuple(diff[0])]!r} oracle "
                               f"{r[tuple(diff[0])]!r}")
    fin = np.isfinite(r)
    assert (~fin).sum() > 0, f"{what}: the injected values gave no non-finite output"
    assert fin.sum() > 0, f"{what}: no finite output left to compare"
    rf, gf = r[fin], g[fin]
    rms = np.sqrt(np.mean(rf * rf))
    bad = np.abs(gf - rf) > 2.0**-7 * np.abs(rf) + 2.0**-10 * rms
    assert not bad.any(), f"{what}: {int(bad.sum())} finite elements outside the tolerance"


def _gemm(sk, x, w, M, splits=0, launch=None):
    import torch

    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if launch is None:
        sk.skinny_gemm_bf16(to_dev(x), to_dev(w), y, splits)
    else:
        sk.skinny_gemm_bf16_launch(to_dev(x), to_dev(w), y, launch)
    torch.cuda.synchronize()
    return from_dev(y)


# (M, N, K, explicit splits): the chooser's launch at each, covering DOT2
# (unpooler 1-4 tokens, o_proj 1 token), the 16-block kernel (unpooler 8-16
# tokens; with 2 splits its in-kernel hand-off), DOT2 with the split reduce
# (unpooler 4 tokens, 2 splits), MFMA with the split reduce (o_proj 16
# tokens, 4 splits), the staged MFMA walk (o_proj 16 tokens) and the DOT2
# and 16-block walks of the full pooler (8 and 16 tokens).
CASES = [(1, 1024, 4096, 0), (4, 1024, 4096, 0), (8, 1024, 4096, 0), (16, 1024, 4096, 0),
         (16, 1024, 4096, 2), (4, 1024, 4096, 2), (1, 8192, 1024, 0), (16, 8192, 1024, 0),
         (16, 8192, 1024, 4), (8, 4096, 8192, 0), (16, 4096, 8192, 0), (12, 512, 8192, 0)]


@pytest.mark.parametrize("M,N,K,splits", CASES)
def test_nonfinite_classes_match_the_oracle(gpu_lib, M, N, K, splits):
    sk = gpu_lib
    l = sk.skinny_choose(M, N, K, splits)
    walk = sk.skinny_choose_walk(M, N, K, splits)
    what = f"M={M} N={N} K={K} S={splits} {l} segment={walk.segment}"
    _say("case", what)
    x, w = _inputs(M, N, K, seed=4242 + M + splits)
    y = _gemm(sk, x, w, M, splits)
    _assert_same_class(y, oracle.gemm_bf16(x, w, THREADS), what)


def test_nonfinite_classes_on_every_path_at_one_shape(gpu_lib):
    """The unpooler shard at 12 tokens through each path's explicit launch:
    DOT2, the 16-x-32 MFMA and the 16-block MFMA, with and without splits."""
    sk = gpu_lib
    M, N, K = 12, 1024, 4096
    x, w = _inputs(M, N, K, seed=77)
    ref = oracle.gemm_bf16(x, w, THREADS)
    launches = [sk.Launch(0, 1, 8, 1, 1, 4), sk.Launch(0, 2, 4, 1, 1, 4),
                sk.Launch(1, 1, 16, 8, 1, 16), sk.Launch(1, 4, 4, 8, 2, 16),
                sk.Launch(3, 1, 8, 4, 1, 8), sk.Launch(3, 1, 8, 4, 2, 8),
                sk.Launch(3, 2, 4, 4, 2, 8)]
    for l in launches:
        why = sk.skinny_launch_unsupported(M, N, K, l)
        assert why is None, f"{l}: {why}"
        _say("launch", l)
        _assert_same_class(_gemm(sk, x, w, M, launch=l), ref, f"{l}")


def test_nonfinite_classes_through_the_ring(gpu_lib):
    """Three independent GEMMs in one ring launch, each with its own
    injected values, at 1 and 16 tokens (DOT2 and 16-block ring kernels)."""
    import torch

    sk = gpu_lib
    N, K = 1024, 4096
    for M in (1, 16):
        xs, ws, ys, refs = [], [], [], []
        for i in range(3):
            x, w = _inputs(M, N, K, seed=900 + 10 * M + i)
            xs.append(to_dev(x))
            ws.append(to_dev(w))
            ys.append(torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))
            refs.append(oracle.gemm_bf16(x, w, THREADS))
        _say("ring M", M, sk.skinny_ring_choose(M, N, K, 3))
        sk.skinny_gemm_bf16_ring(xs, ws, ys)
        torch.cuda.synchronize()
        for i in range(3):
            _assert_same_class(from_dev(ys[i]), refs[i], f"ring M={M} item {i}")
