"""Pins for the oracle GEMM y = bf16(x @ W^T) (unpooler page, module
description: BF16 operands and result, sums in FP32 or wider, 1 to 16
tokens).

Pins: exact rational brute force on tiny inputs, closed forms (identity,
one-hot, power-of-two scaling), numpy's float64 matmul on the exact sums, and
integer inputs whose result is exact in any order.  A transposed operand, a
dropped term or a wrong index fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from tests.test_oracle_formats import _nearest_bf16_bits_exact


def _bf16(bits):
    return oracle.bf16_value(bits)


@pytest.mark.parametrize("seed", range(12))
def test_gemm_brute_force_rational(seed):
    rng = np.random.default_rng(seed)
    M, N, K = rng.integers(1, 5, 3)
    x = synthetic.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = synthetic.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    y = oracle.gemm_bf16(x, w)
    xv, wv = _bf16(x), _bf16(w)
    for m in range(M):
        for n in range(N):
            s = sum(Fraction(float(xv[m, k])) * Fraction(float(wv[n, k])) for k in range(K))
            assert int(y[m, n]) == _nearest_bf16_bits_exact(s)


def test_gemm_midpoint_ties():
    # y = a * 1 + b * 1 where a + b is exactly halfway between two bf16
    # numbers: the oracle must round the exact sum once, to even.
    a = np.float32(1.0)
    b = np.float32(2.0**-8)  # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7
    x = synthetic.to_bf16_bits(np.array([[a, b], [a, 3 * b]], dtype=np.float32))
    w = synthetic.to_bf16_bits(np.array([[1.0, 1.0]], dtype=np.float32))
    y = oracle.gemm_bf16(x, w)
    assert int(y[0, 0]) == 0x3F80  # 1 + 2^-8 -> 1.0 (even)
    assert int(y[1, 0]) == 0x3F82  # 1 + 3*2^-8 -> 1 + 2^-6 (even)


def test_gemm_identity_and_one_hot():
    rng = np.random.default_rng(5)
    K = 40
    x = synthetic.to_bf16_bits(rng.standard_normal((3, K)).astype(np.float32))
    eye = synthetic.to_bf16_bits(np.eye(K, dtype=np.float32))
    assert np.array_equal(oracle.gemm_bf16(x, eye), x)
    # one-hot x rows pick columns of W: y[m, n] = W[n, k_m]
    N = 24
    w = synthetic.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    ks = [0, 17, K - 1]
    onehot = np.zeros((3, K), dtype=np.float32)
    for m, k in enumerate(ks):
        onehot[m, k] = 1.0
    y = oracle.gemm_bf16(synthetic.to_bf16_bits(onehot), w)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], w[:, k])


def test_gemm_power_of_two_scaling():
    x, w = synthetic.gemm_inputs(N=32, K=64, seed=6)
    y = oracle.gemm_bf16(x[:4], w)
    xs = synthetic.to_bf16_bits((_bf16(x[:4]) * 8.0).astype(np.float32))
    y8 = oracle.gemm_bf16(xs, w)
    assert np.array_equal(_bf16(y8), _bf16(y) * 8.0)


def test_gemm_exact_sums_match_numpy_float64():
    x, w = synthetic.gemm_inputs(N=48, K=256, seed=7)
    M = 5
    rows, cols = np.meshgrid(np.arange(M), np.arange(48), indexing="ij")
    _, exact = oracle.gemm_bf16_sampled(x[:M], w, rows.ravel(), cols.ravel())
    ref = _bf16(x[:M]) @ _bf16(w).T
    np.testing.assert_allclose(exact.reshape(M, 48), ref, rtol=1e-12, atol=1e-12)
    # and the full GEMM rounds those sums
    y = oracle.gemm_bf16(x[:M], w)
    assert np.array_equal(y.ravel(), oracle.bf16_round(exact))


def test_gemm_non_square_orientation():
    # x [2, 3], W [4, 3]: y[m, n] = sum_k x[m, k] W[n, k]; any transposition of
    # an operand changes the shape or the values.
    x = synthetic.to_bf16_bits(np.array([[1, 2, 3], [4, 5, 6]], dtype=np.float32))
    w = synthetic.to_bf16_bits(np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1]],
                                        dtype=np.float32))
    y = _bf16(oracle.gemm_bf16(x, w))
    assert y.shape == (2, 4)
    assert np.array_equal(y, np.array([[1, 2, 3, 6], [4, 5, 6, 15]], dtype=np.float64))


def test_gemm_exact_integer_inputs():
    x, w = synthetic.exact_integer_inputs(M=16, N=64, K=512, seed=8)
    y = _bf16(oracle.gemm_bf16(x, w))
    ref = _bf16(x).astype(np.int64) @ _bf16(w).astype(np.int64).T
    assert np.abs(ref).max() <= 256
    assert np.array_equal(y, ref.astype(np.float64))


def test_gemm_threads_do_not_change_result():
    x, w = synthetic.gemm_inputs(N=64, K=512, seed=9)
    assert np.array_equal(oracle.gemm_bf16(x, w, threads=1), oracle.gemm_bf16(x, w, threads=4))


def test_gemm_sampled_matches_full():
    x, w = synthetic.gemm_inputs(N=80, K=96, seed=10)
    y = oracle.gemm_bf16(x, w)
    rng = np.random.default_rng(0)
    r = rng.integers(0, 16, 50)
    c = rng.integers(0, 80, 50)
    got, _ = oracle.gemm_bf16_sampled(x, w, r, c)
    assert np.array_equal(got, y[r, c])
