"""Constructed inputs for the norm -> NVFP4 parity tests: rows whose normed
values land exactly on every rounding boundary of the two NVFP4 formats
(pooler_gather page: cvt_e2m1x8_f32 and cvt_f32_to_e4m3 round to nearest
even with saturation; nvfp4_compute_output_scale), on subnormal block scales,
and on signed zeros.

The construction holds no arithmetic of the method.  Every row r is +-1 in
every column and the norm runs with eps = 0 and gain center 0, so the mean
square is exactly 1, the reciprocal root exactly 1 and the normed value is
exactly r_j * w_j: the norm weight w then places each normed value where it
is wanted.  The block scale is e4m3(global_scale * amax / 6), so
  - with global_scale 1 and a block amax of 6 the output scale is exactly 1
    and the normed values themselves meet the e2m1 midpoints;
  - with global_scale 6 the unrounded block scale equals the block amax, so
    a block whose amax is an e4m3 midpoint is an exact e4m3 tie.
tests/test_norm_cases.py checks through the oracle that each case really
reaches the points it is built for.
"""
from __future__ import annotations

import numpy as np

import synthetic

E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _bits(values) -> np.ndarray:
    """float64 values that are exactly bfloat16 -> their bit patterns."""
    v = np.asarray(values, dtype=np.float64)
    bits = synthetic.to_bf16_bits(v.astype(np.float32))
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    same = (back == v) & (np.signbit(back) == np.signbit(v))
    if not np.all(same):
        raise ValueError(f"not a bfloat16 value: {v[~same][:4]}")
    return bits


def _step(bits: np.ndarray, d: int) -> np.ndarray:
    """The bfloat16 neighbour d patterns away (same sign, nonzero values)."""
    return (bits.astype(np.int32) + d).astype(np.uint16)


def _sign_rows(P: int, seed: int) -> np.ndarray:
    """Three +-1 rows: all +1, all -1, random signs."""
    rng = np.random.default_rng(seed)
    rows = np.ones((3, P))
    rows[1] = -1.0
    rows[2] = np.where(rng.random(P) < 0.5, -1.0, 1.0)
    return _bits(rows)


def e2m1_tie_case():
    """Returns (r_bits [3, P], w_bits [P], gain_center, eps, global_scale).

    Blocks (16 columns each):
      0  amax 6 (output scale 1): every e2m1 midpoint, both signs, and -0.125
      1  the same with each midpoint moved one bfloat16 step up
      2  ... and one step down
      3  amax 3 (block scale 0.5, output scale 2): the midpoints halved
      4  amax 6.375 (unrounded scale 1.0625, an e4m3 tie kept at 1.0): values
         above 6 saturate to code 7
      5  signed zeros: -0.0, +0.0, tiny negatives that round to code 0x8
      6  amax below the smallest half e4m3 step: scale code 0, output scale 0,
         every code a bare sign
      7  amax exactly half the smallest e4m3 subnormal (ties to scale code 0)
    """
    m = np.array(E2M1_MIDPOINTS)
    b0 = np.concatenate([[6.0], m, -m, [-0.125]])
    b0_bits = _bits(b0)
    b1_bits = b0_bits.copy()
    b1_bits[1:15] = _step(b0_bits[1:15], +1)
    b2_bits = b0_bits.copy()
    b2_bits[1:15] = _step(b0_bits[1:15], -1)
    b3 = np.concatenate([[3.0], m / 2, -m / 2, [-0.0625]])
    b4 = np.array([6.375, -6.375, 6.25, 6.125, 5.5, 5.0, -5.0, 4.5, 3.5, 0.75,
                   -0.25, 0.25, 1.75, -1.25, 2.5, 0.0])
    b5 = np.array([6.0, -0.0, 0.0, -0.125, -0.25, -2.0 ** -20, 0.125, -0.0,
                   0.0, -0.0, -1.0, 1.0, -0.5, 0.5, -2.0 ** -100, 2.0 ** -100])
    b6 = np.array([-2.0 ** -9, 2.0 ** -9, -0.0, 0.0, -2.0 ** -12, 2.0 ** -12, -2.0 ** -20,
                   2.0 ** -20, -2.0 ** -9, -2.0 ** -10, 2.0 ** -10, -2.0 ** -11,
                   -2.0 ** -30, 0.0, -0.0, 2.0 ** -9])
    # 6 * 2^-10 / 6 = 2^-10 = half of the smallest subnormal 2^-9: ties to 0
    b7 = np.array([6.0 * 2.0 ** -10] + [-2.0 ** -11] * 5 + [2.0 ** -12] * 10)
    w = np.concatenate([b0_bits, b1_bits, b2_bits, _bits(b3), _bits(b4), _bits(b5),
                        _bits(b6), _bits(b7)])
    r = _sign_rows(w.size, seed=21)
    return r, w, 0.0, 0.0, 1.0


def e4m3_midpoints() -> np.ndarray:
    """Midpoints between consecutive finite non-negative e4m3fn values,
    from the format definition (bias 7, 3 mantissa bits, subnormal step
    2^-9, largest finite 448), plus the midpoint 464 between 448 and the
    next binade step, where saturation takes over."""
    vals = [m * 2.0 ** -9 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                break
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    vals = np.array(vals)
    assert vals[-1] == 448.0 and vals.size == 127
    mids = (vals[:-1] + vals[1:]) / 2
    return np.concatenate([mids, [464.0]]), vals


def e4m3_tie_case():
    """Returns (r_bits [3, P], w_bits [P], gain_center, eps, global_scale).

    global_scale 6, so the unrounded block scale is exactly the block amax.
    One block per amax in: every e4m3 midpoint (126 inside the range and
    464), every finite nonzero e4m3 value (exact scales 0x01..0x7E), and
    values past the range (480, 512, 1024, 2^20) that saturate to 0x7E.  The
    other 15 values of a block are fixed fractions of its amax, of both signs
    and of at most three significant bits, so that every product is still a
    bfloat16 value."""
    mids, vals = e4m3_midpoints()
    amaxes = np.concatenate([mids, vals[1:], [480.0, 512.0, 1024.0, 2.0 ** 20]])
    frac = np.array([-1.0, 0.5, -0.5, 0.75, -0.75, 0.25, 0.375, -0.625, 0.875,
                     -0.125, 0.0625, -0.875, 0.3125, 0.0, -0.0])
    blocks = [np.concatenate([[a], a * frac]) for a in amaxes]
    w = _bits(np.concatenate(blocks))
    r = _sign_rows(w.size, seed=22)
    return r, w, 0.0, 0.0, 6.0


def subnormal_scale_case(gs_target: float = 2.0 ** -6, M: int = 8, P: int = 4096, seed: int = 5):
    """Normal rows whose global scale puts the row set's largest block scale
    near `gs_target`; with the default 2^-6 (the smallest normal e4m3 value)
    nearly every block scale is an e4m3 subnormal.  Returns (r_bits, w_bits,
    gain_center, eps, global_scale as a function of the oracle's yn)."""
    r = synthetic.rows_normal(M, P, seed=seed)
    w = synthetic.norm_weight(P, seed=seed)

    def global_scale(yn_values: np.ndarray) -> float:
        return float(np.float32(6.0 * gs_target / np.abs(yn_values).max()))

    return r, w, 1.0, 1e-6, global_scale
