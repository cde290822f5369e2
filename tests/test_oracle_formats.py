"""Pins for the oracle's number formats: bfloat16 rounding, e4m3fn and e2m1.

Each pin comes from outside the oracle: a library routine (torch's float32 ->
bfloat16 and float8_e4m3fn conversions), an exact rational computation, an
exhaustive nearest-value search written here, or the format definitions.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _to_f32_quiet(v):
    with np.errstate(over="ignore"):
        return v.astype(np.float32)


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # the signalling-NaN patterns widen to NaN
        vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits, vals


def _nearest_bf16_bits_exact(v: Fraction) -> int:
    """Brute-force round-to-nearest-even to bfloat16 with exact rationals:
    the two finite neighbours from a sorted table of every finite pattern."""
    bits, vals = _all_bf16_values()
    finite = np.isfinite(vals)
    pos = (bits < 0x8000) & finite
    pb, pv = bits[pos], vals[pos]
    order = np.argsort(pv, kind="stable")
    pb, pv = pb[order], pv[order]
    a = abs(v)
    sign = 0x8000 if v < 0 else 0
    i = int(np.searchsorted(pv, float(a)))
    cands = set()
    for j in (i - 2, i - 1, i, i + 1):
        if 0 <= j < len(pv):
            cands.add(j)
    best = None
    for j in sorted(cands):
        d = abs(Fraction(float(pv[j])) - a)
        key = (d, int(pb[j]) & 1)  # tie -> even last bit
        if best is None or key < best[0]:
            best = (key, int(pb[j]))
    # beyond the largest finite value by at least half an ulp -> infinity
    top = Fraction(float(pv[-1]))
    ulp = Fraction(2) ** (127 - 7)
    if a >= top + ulp / 2:
        return sign | 0x7F80
    return sign | best[1]


def test_bf16_roundtrip_every_pattern():
    bits, vals = _all_bf16_values()
    finite = np.isfinite(vals)
    back = oracle.bf16_round(vals[finite])
    assert np.array_equal(back, bits[finite])


def test_bf16_round_matches_torch_from_float32():
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even; on
    # float32 inputs a single rounding from binary64 must agree with it.
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-38).astype(np.float32),  # subnormal
        # large values: some overflow to +-Inf in float32 on purpose
        _to_f32_quiet(rng.standard_normal(5000) * 1e38),
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    f = np.concatenate(parts)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_exact_rational_midpoints():
    rng = np.random.default_rng(2)
    bits, vals = _all_bf16_values()
    idx = rng.integers(0, 0x7F7F, 300)
    cases = []
    for i in idx:
        lo = Fraction(float(vals[i]))
        hi = Fraction(float(vals[i + 1]))
        mid = (lo + hi) / 2
        cases += [mid, -mid]
        eps = Fraction(1, 2**60) * (hi - lo) * 2**50
        cases += [mid + eps, mid - eps]
    cases += [Fraction(float(v) * 7.59375) for v in rng.standard_normal(200)]
    for c in cases:
        got = int(oracle.bf16_round(np.float64(float(c)))[()])
        # every case is exactly representable in binary64
        assert Fraction(float(c)) == c
        assert got == _nearest_bf16_bits_exact(c), float(c)


def test_bf16_round_specials():
    assert int(oracle.bf16_round(np.float64(2.0**128))) == 0x7F80
    assert int(oracle.bf16_round(np.float64(-(2.0**128)))) == 0xFF80
    big = float((Fraction(255, 128) + Fraction(1, 256)) * 2**127)  # halfway above max
    assert int(oracle.bf16_round(np.float64(big))) == 0x7F80
    assert int(oracle.bf16_round(np.float64(-0.0))) == 0x8000
    assert int(oracle.bf16_round(np.float64(2.0**-134))) == 0x0000  # tie to even zero
    assert int(oracle.bf16_round(np.float64(3 * 2.0**-135))) == 0x0001


# ---------------------------------------------------------------- e4m3fn
def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_e4m3_encode_matches_torch_in_range():
    # torch rounds to nearest even and gives NaN past 464 (no saturation);
    # within |v| <= 464 the two must agree, beyond it the oracle saturates.
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.uniform(-464, 464, 20000),
        rng.standard_normal(20000) * 0.02,
        rng.standard_normal(5000) * 1e-3,
    ]).astype(np.float32)
    # every midpoint between adjacent finite codes, and +-1 float32 ulp
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    v = v[np.abs(v) <= 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(t)) for t in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_saturates_and_roundtrips():
    for v in (464.0001, 480.0, 1000.0, 1e30, float("inf")):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c
    assert oracle.e4m3_encode(float("nan")) == 0x7F


# ------------------------------------------------------------------ e2m1
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the format's table


def test_e2m1_decode_table():
    for c in range(16):
        mag = E2M1_MAGNITUDES[c & 7]
        assert oracle.e2m1_value(c) == (-mag if c & 8 else mag)


@pytest.mark.parametrize(
    "v,code",
    [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6),
     (5.0, 0x6), (6.0, 0x7), (7.0, 0x7), (1e9, 0x7), (0.2500001, 0x1), (0.2499999, 0x0),
     (-0.25, 0x8), (-0.0, 0x8), (0.0, 0x0), (-5.0, 0xE), (-100.0, 0xF)],
)
def test_e2m1_ties_and_saturation(v, code):
    assert oracle.e2m1_encode(v) == code


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(4)
    vals = np.concatenate([rng.uniform(-8, 8, 20000), rng.standard_normal(2000) * 0.3])
    mags = np.array(E2M1_MAGNITUDES)
    for v in vals:
        d = np.abs(abs(v) - mags)
        best = int(np.argmin(d))  # argmin takes the first (smaller index) on ties
        ties = np.flatnonzero(d == d[best])
        if len(ties) > 1:
            best = int([t for t in ties if t % 2 == 0][0])
        expect = (0x8 if np.signbit(v) else 0) | best
        assert oracle.e2m1_encode(float(v)) == expect
