"""The constructed norm -> NVFP4 cases reach the points they are built for
(tests/norm_cases.py), checked through the oracle on the CPU, so that the GPU
parity tests on them really compare the kernel at every rounding boundary.

Format facts used here come from the format definitions (e2m1 magnitudes
0, 0.5, 1, 1.5, 2, 3, 4, 6; e4m3fn bias 7 with 3 mantissa bits, subnormal
step 2^-9, largest finite 448), not from the oracle's code."""
import numpy as np

import oracle
from tests import norm_cases
from tests.helpers import unpack_codes


def test_e2m1_case_meets_every_midpoint_both_signs():
    r, w, gc, eps, gs = norm_cases.e2m1_tie_case()
    ref = oracle.rmsnorm_nvfp4(r, w, gc, eps, gs)
    pre = ref["pre"]
    for m in norm_cases.E2M1_MIDPOINTS:
        assert (pre == m).sum() >= 3 and (pre == -m).sum() >= 3, m
    # the normed values are exactly r * (w + 0) (mean square 1, eps 0, gain
    # center 0; w + 0 turns a -0.0 weight into +0.0, so a zero takes r's sign)
    yn = oracle.bf16_value(ref["yn"])
    want = oracle.bf16_value(r) * (oracle.bf16_value(w)[None, :] + 0.0)
    assert np.array_equal(yn, want)
    assert np.array_equal(np.signbit(yn), np.signbit(want))


def test_e2m1_case_scales_and_signed_zeros():
    r, w, gc, eps, gs = norm_cases.e2m1_tie_case()
    ref = oracle.rmsnorm_nvfp4(r, w, gc, eps, gs)
    # block scales: 1.0 = 0x38 (exp 7), 0.5 = 0x30, and code 0 for blocks 6, 7
    assert ref["a_sf"].tolist() == [[0x38, 0x38, 0x38, 0x30, 0x38, 0x38, 0, 0]] * 3
    codes = unpack_codes(ref["a"])
    yn = oracle.bf16_value(ref["yn"])
    neg_zero = (yn == 0) & np.signbit(yn)
    assert neg_zero.sum() >= 6
    # negative values that round to zero, -0.0 itself among them, keep the sign
    tiny_neg = np.signbit(yn) & (np.abs(yn) * ref["os"].repeat(16, axis=1) <= 0.25)
    assert tiny_neg.sum() >= 12 and np.all(codes[tiny_neg] == 0x8)
    # the zero-scale blocks hold bare signs only
    assert np.all((codes[:, 96:128] & 7) == 0) and np.any(codes[:, 96:128] == 8)
    # values above 6 at output scale 1 saturate to magnitude index 7
    assert np.all(codes[0, 64:66] & 7 == 7)


def test_e4m3_case_ties_every_scale_midpoint():
    r, w, gc, eps, gs = norm_cases.e4m3_tie_case()
    mids, vals = norm_cases.e4m3_midpoints()
    ref = oracle.rmsnorm_nvfp4(r, w, gc, eps, gs)
    sf = ref["a_sf"]
    yn = oracle.bf16_value(ref["yn"][0])
    amax = np.abs(yn.reshape(-1, 16)).max(axis=1)
    n = mids.size
    # the unrounded block scale gs * amax / 6 is exactly each midpoint
    assert np.array_equal(gs * amax[:n] / 6.0, mids)
    # every code 0x00..0x7E occurs, and 0x7E for all saturating blocks
    assert sorted(set(sf[0].tolist())) == list(range(0x7F))
    assert np.all(sf[:, -4:] == 0x7E) and np.all(sf[:, n - 1] == 0x7E)
    # the two neighbours of each tie: the result is one of them, and the even one
    lo_code = np.searchsorted(vals, mids[:-1]) - 1
    got = sf[0, : n - 1].astype(int)
    assert np.all((got == lo_code) | (got == lo_code + 1))
    assert np.all(got % 2 == 0)
    # the exact e4m3 values map to themselves (codes 1..0x7E)
    assert np.array_equal(sf[0, n : n + 126], np.arange(1, 0x7F))


def test_subnormal_case_has_every_subnormal_scale():
    r, w, gc, eps, gs_of = norm_cases.subnormal_scale_case()
    yn = oracle.bf16_value(oracle.rmsnorm_bf16(r, w, gc, eps))
    gs = gs_of(yn)
    ref = oracle.rmsnorm_nvfp4(r, w, gc, eps, gs)
    codes = set(ref["a_sf"].ravel().tolist())
    assert set(range(1, 9)) <= codes and max(codes) == 8
    frac_sub = np.mean((ref["a_sf"] >= 1) & (ref["a_sf"] <= 7))
    assert frac_sub > 0.9
