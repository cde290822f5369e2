"""Pins for the oracle's RMSNorm and NVFP4 quantizer (pooler_gather page:
module description, cvt_e2m1x8_f32, cvt_f32_to_e4m3,
nvfp4_compute_output_scale).

Pins: the hand-worked blocks in tests/golden/nvfp4_worked.txt, closed forms
for constant and one-hot rows, the global-max-block invariant, the all-zero
block, and the dequantization error bound.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_worked.txt")


def _parse_golden():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, *fields = line.split()
            kv = dict(fld.split("=", 1) for fld in fields)
            cases.append((kind, kv))
    return cases


def _floats(s):
    return [float(t) for t in s.split(",")]


def _hex(s):
    return [int(t, 16) for t in s.split(",")]


@pytest.mark.parametrize("case", _parse_golden(), ids=lambda c: c[0])
def test_golden_worked_blocks(case):
    kind, kv = case
    expect_a = np.array(_hex(kv["a"]), dtype=np.uint8)
    expect_sf = int(kv["sf"], 16)
    if kind == "norm":
        r = synthetic.to_bf16_bits(np.array([_floats(kv["r"])], dtype=np.float32))
        w = synthetic.to_bf16_bits(np.full(16, float(kv["w"]), dtype=np.float32))
        out = oracle.rmsnorm_nvfp4(r, w, float(kv["gc"]), float(kv["eps"]), float(kv["gs"]))
        assert np.array_equal(out["a"][0], expect_a)
        assert int(out["a_sf"][0, 0]) == expect_sf
    else:
        codes, sf, _, _ = oracle.nvfp4_block(np.array(_floats(kv["yn"])), float(kv["gs"]))
        packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        assert np.array_equal(packed, expect_a)
        assert sf == expect_sf


def test_rmsnorm_constant_row_closed_form():
    # r_j = c for all j: mean(r^2) = c^2, so yn_j = bf16(c / sqrt(c^2 + eps) * g_j)
    P, c, eps, gc = 256, 0.75, 1e-2, 1.0
    r = synthetic.to_bf16_bits(np.full((1, P), c, dtype=np.float32))
    w = synthetic.norm_weight(P, seed=1)
    yn = oracle.bf16_value(oracle.rmsnorm_bf16(r, w, gc, eps))[0]
    g = oracle.bf16_value(w) + gc
    scale = c / math.sqrt(c * c + oracle.f32(eps))
    expect = oracle.bf16_value(oracle.bf16_round(scale * g))
    assert np.array_equal(yn, expect)


def test_rmsnorm_one_hot_closed_form():
    # r = a e_j: mean(r^2) = a^2 / P, yn_j = bf16(a sqrt(P) / sqrt(a^2 + P eps) g_j)
    P, a, j, eps, gc = 512, 3.0, 77, 1e-6, 1.0
    row = np.zeros((1, P), dtype=np.float32)
    row[0, j] = a
    w = synthetic.norm_weight(P, seed=2)
    yn = oracle.bf16_value(oracle.rmsnorm_bf16(synthetic.to_bf16_bits(row), w, gc, eps))[0]
    g = oracle.bf16_value(w)[j] + gc
    e = oracle.f32(eps)
    expect = oracle.bf16_value(oracle.bf16_round(a * math.sqrt(P) / math.sqrt(a * a + P * e) * g))
    assert yn[j] == expect
    assert np.all(yn[np.arange(P) != j] == 0.0)


def test_rmsnorm_nvfp4_agrees_with_rmsnorm_bf16():
    r = synthetic.rows_normal(3, 128, seed=3)
    w = synthetic.norm_weight(128, seed=3)
    yn = oracle.rmsnorm_bf16(r, w, 1.0, 1e-6)
    out = oracle.rmsnorm_nvfp4(r, w, 1.0, 1e-6, 100.0)
    assert np.array_equal(out["yn"], yn)


def test_global_max_block_hits_the_largest_codes():
    # with global_scale = 448 * 6 / amax(yn), the block holding the row-set
    # maximum gets sf = 448 (0x7E) and its maximum element code index 7.
    r = synthetic.rows_normal(4, 1024, seed=4)
    w = synthetic.norm_weight(1024, seed=4)
    yn = oracle.bf16_value(oracle.rmsnorm_bf16(r, w, 1.0, 1e-6))
    amax = np.abs(yn).max()
    gs = oracle.f32(448.0 * 6.0 / amax)
    out = oracle.rmsnorm_nvfp4(r, w, 1.0, 1e-6, gs)
    m, col = np.unravel_index(np.argmax(np.abs(yn)), yn.shape)
    b = col // 16
    assert out["a_sf"][m, b] == 0x7E
    byte = out["a"][m, col // 2]
    code = (byte >> 4) if col % 2 else (byte & 0xF)
    assert code & 7 == 7
    # no scale exceeds 448 and none is NaN
    assert np.all((out["a_sf"] & 0x7F) <= 0x7E)


def test_all_zero_block():
    P = 64
    r = np.zeros((1, P), dtype=np.float32)
    r[0, 32:] = 1.0  # blocks 0 and 1 are zero, 2 and 3 are not
    w = synthetic.to_bf16_bits(np.full(P, 0.5, dtype=np.float32))
    out = oracle.rmsnorm_nvfp4(synthetic.to_bf16_bits(r), w, 1.0, 1e-6, 50.0)
    assert np.all(out["a_sf"][0, :2] == 0)
    assert np.all(out["a"][0, :16] == 0)
    assert np.all(out["os"][0, :2] == 0.0)
    assert np.all(out["a_sf"][0, 2:] != 0)


def test_dequantization_error_bound():
    # outside saturation, |dec(q) - yn * os| <= half the e2m1 step at that
    # magnitude, i.e. |dec(q) / os - yn| <= step / 2 / os
    r = synthetic.rows_normal(8, 4096, seed=5)
    w = synthetic.norm_weight(4096, seed=5)
    yn_bits = oracle.rmsnorm_bf16(r, w, 1.0, 1e-6)
    yn = oracle.bf16_value(yn_bits)
    gs = oracle.f32(2688.0 / np.abs(yn).max())
    out = oracle.rmsnorm_nvfp4(r, w, 1.0, 1e-6, gs)
    lo = out["a"] & 0xF
    hi = out["a"] >> 4
    codes = np.empty(yn.shape, dtype=np.uint8)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    table = np.array([oracle.e2m1_value(c) for c in range(16)])
    deq = table[codes]
    pre = out["pre"]
    mag = np.abs(pre)
    step = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
    unsat = mag <= 6
    assert np.all(np.abs(deq - pre)[unsat] <= step[unsat] / 2 + 1e-12)
    # pre = yn * os with os = gs / dec(sf)
    sf_val = np.array([[oracle.e4m3_value(c) for c in row] for row in out["a_sf"]])
    os_ = np.where(sf_val == 0, 0.0, gs / np.where(sf_val == 0, 1, sf_val))
    np.testing.assert_array_equal(out["os"], os_)
    np.testing.assert_allclose(pre, yn * np.repeat(os_, 16, axis=1), rtol=0, atol=0)


def test_packing_low_nibble_even_column():
    # one block whose codes are all distinct: the packed byte i must hold code
    # 2i in its low nibble and code 2i + 1 in its high nibble
    yn = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 0.0])
    codes, sf, _, _ = oracle.nvfp4_block(yn, global_scale=6.0)  # amax 6 -> s = 6 -> os 1
    assert sf == oracle.e4m3_encode(6.0)
    assert list(codes) == [0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 0]
