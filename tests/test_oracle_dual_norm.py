"""Pins of the oracle's dual norm (post_attn_norm -> gated FP32 residual add
-> pre_ffn_norm; oproj.batt page, AttentionBoundary).

The pages fix only the order of the steps, the dtypes (BF16 partial and
output, FP32 stream updated in place) and the parameters (optional post
weight, alpha as a tensor or a float, beta, next weight).  The formula of the
gated add and the rounding points are a reading of the pages (stated in the oracle
source): these pins check the oracle against closed forms of that reading,
so a slip in it (a dropped term, swapped constants, the wrong stream fed to
the second norm) fails; whether the reading is the pages' own stays unpinned.
"""
import math

import numpy as np
import pytest

import oracle
import synthetic

H = 64


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, dtype=np.float64))


def _val(bits):
    return oracle.bf16_value(bits)


def _rand_w(seed, scale=0.3):
    rng = np.random.default_rng(seed)
    return _bf16(rng.normal(0.0, scale, H))


def test_identity_gate_keeps_stream_and_normalises_it():
    """alpha = 1, beta = 0: the stream is unchanged bit for bit and out is the
    pre norm of a constant row: bf16(c / sqrt(c^2 + eps) * (w + gc))."""
    c, eps, gc = 0.1, 1e-2, 1.0  # eps comparable to c^2, so it shows in the output
    partial = _bf16(np.random.default_rng(1).normal(size=(2, H)))
    stream = np.full((2, H), c, dtype=np.float32)
    nw = _rand_w(2)
    out, st, _ = oracle.dual_norm(partial, stream, _rand_w(3), 0.5, 1e-6, 1.0, _bf16(np.zeros(H)),
                                  nw, gc, eps)
    assert np.array_equal(st, stream)
    eps32 = float(np.float32(eps))
    want = oracle.bf16_round(c / math.sqrt(c * c + eps32) * (_val(nw) + gc))
    assert np.array_equal(out, np.broadcast_to(want, (2, H)))


def test_beta_gate_replaces_stream_with_post_norm():
    """alpha = 0, beta = 1: the stream becomes the post norm of a constant
    partial row, bf16(c / sqrt(c^2 + eps) * (w + gc)), exactly."""
    c, eps, gc = -2.0, 0.25, 0.5
    partial = _bf16(np.full((1, H), c))
    pw = _rand_w(4)
    out, st, h = oracle.dual_norm(partial, np.full((1, H), 7.0, np.float32), pw, gc, eps, 0.0,
                                  _bf16(np.ones(H)), _rand_w(5), 1.0, 1e-6)
    want_h = oracle.bf16_round(c / math.sqrt(c * c + eps) * (_val(pw) + gc))
    assert np.array_equal(h[0], want_h)
    assert np.array_equal(st[0], _val(want_h).astype(np.float32))


def test_post_norm_without_weight_one_hot():
    """No post weight (scale 1): a one-hot partial a * e_k normalises to
    a * sqrt(H) / sqrt(a^2 + H eps) at k and zero elsewhere."""
    a, k, eps = 5.0, 7, 1e-2
    p = np.zeros((1, H))
    p[0, k] = a
    _, st, h = oracle.dual_norm(_bf16(p), np.zeros((1, H), np.float32), None, 123.0, eps, 0.0,
                                _bf16(np.ones(H)), _rand_w(6), 1.0, 1e-6)
    eps32 = float(np.float32(eps))
    want = oracle.bf16_round(a * math.sqrt(H) / math.sqrt(a * a + H * eps32))
    assert h[0, k] == want and np.all(_val(np.delete(h[0], k)) == 0.0)
    assert st[0, k] == np.float32(_val(want))


@pytest.mark.parametrize("alpha_per_channel", [False, True])
def test_gated_add_exact_small_numbers(alpha_per_channel):
    """eps = 0 and a constant partial row c > 0 make h = g exactly (g = w + gc
    representable); the gated add on small binary numbers is then exact:
    stream = alpha * s + beta * g."""
    rng = np.random.default_rng(7)
    g = rng.integers(-4, 5, H).astype(np.float64)
    s = rng.integers(-8, 9, (1, H)).astype(np.float32)
    beta = rng.choice([0.0, 0.5, 1.0, -2.0], H)
    alpha = rng.choice([1.0, 2.0, -0.5], H) if alpha_per_channel else 2.0
    _, st, h = oracle.dual_norm(_bf16(np.full((1, H), 3.0)), s, _bf16(g), 0.0, 0.0,
                                _bf16(alpha) if alpha_per_channel else alpha, _bf16(beta),
                                _rand_w(8), 1.0, 1e-6)
    assert np.array_equal(_val(h[0]), g)
    want = (np.asarray(alpha) * s[0].astype(np.float64) + beta * g).astype(np.float32)
    assert np.array_equal(st[0], want)


def test_pre_norm_reads_the_updated_stream():
    """With alpha = 0 and beta = 1 the output is the pre norm of h, so it does
    not depend on the stream that came in."""
    partial = _bf16(np.random.default_rng(9).normal(size=(3, H)))
    args = (_rand_w(10), 1.0, 1e-6, 0.0, _bf16(np.ones(H)), _rand_w(11), 0.25, 1e-5)
    out1, _, _ = oracle.dual_norm(partial, np.zeros((3, H), np.float32), args[0], *args[1:])
    out2, _, _ = oracle.dual_norm(partial, np.full((3, H), 9.0, np.float32), args[0], *args[1:])
    assert np.array_equal(out1, out2)


def test_rows_are_independent():
    rng = np.random.default_rng(12)
    partial = _bf16(rng.normal(size=(4, H)))
    stream = rng.normal(size=(4, H)).astype(np.float32)
    args = (_rand_w(13), 1.0, 1e-6, 0.75, _rand_w(14), _rand_w(15), 1.0, 1e-6)
    out, st, _ = oracle.dual_norm(partial, stream, *args)
    perm = [2, 0, 3, 1]
    out_p, st_p, _ = oracle.dual_norm(partial[perm], stream[perm], *args)
    assert np.array_equal(out_p, out[perm]) and np.array_equal(st_p, st[perm])
