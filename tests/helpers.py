"""Shared helpers for the GPU parity tests: device transfer of bfloat16 bit
patterns and the acceptance rules.

GEMM rule (written in the tests, from the decode GEMM's precision: BF16 out,
FP32 accumulation):  for every element
    |y_gpu - y_ref| <= 2^-7 |y_ref| + 2^-10 rms(y_ref)
evaluated in float64, with rms over all M*N elements of that call; NaN and
Inf fail.  y_ref is the oracle's single rounding of the exact sum, y_gpu the
kernel's rounding of an FP32 sum, so they may differ by one bf16 ulp near a
rounding midpoint (1 ulp <= 2^-7 relative).

NVFP4 rule: codes and scales bit-exact, except where the oracle's value lies
within one bfloat16 ulp (scaled) of a rounding boundary of the target format.
"""
from __future__ import annotations

import numpy as np

import oracle


def to_dev(bits: np.ndarray, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_dev(t) -> np.ndarray:
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def gemm_tolerance_failures(y_gpu_bits: np.ndarray, y_ref_bits: np.ndarray):
    """Indices of elements outside |err| <= 2^-7 |ref| + 2^-10 rms(ref)."""
    g = oracle.bf16_value(y_gpu_bits)
    r = oracle.bf16_value(y_ref_bits)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    bad = ~np.isfinite(g) | (np.abs(g - r) > 2.0**-7 * np.abs(r) + 2.0**-10 * rms)
    return np.argwhere(bad)


def assert_gemm_close(y_gpu_bits, y_ref_bits, what=""):
    bad = gemm_tolerance_failures(y_gpu_bits, y_ref_bits)
    if len(bad):
        i = tuple(bad[0])
        g = oracle.bf16_value(y_gpu_bits)[i]
        r = oracle.bf16_value(y_ref_bits)[i]
        raise AssertionError(f"{what}: {len(bad)} of {y_ref_bits.size} outside tolerance; "
                             f"first at {i}: gpu {g!r} oracle {r!r}")


def bf16_ulp(values: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |values| (float64 in, float64 out)."""
    v = np.abs(np.asarray(values, dtype=np.float64))
    out = np.full(v.shape, 2.0**-133)
    nz = v >= 2.0**-126
    e = np.floor(np.log2(v[nz]))
    out[nz] = 2.0 ** (e - 7)
    return out


E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _e4m3_midpoints():
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    return (vals[:-1] + vals[1:]) / 2


def _interval_has(mids, lo, hi):
    return np.any((mids[None, :] >= lo[:, None]) & (mids[None, :] <= hi[:, None]), axis=1)


def unpack_codes(a: np.ndarray) -> np.ndarray:
    """[M, P/2] packed bytes -> [M, P] 4-bit codes (even column = low nibble)."""
    codes = np.empty((a.shape[0], a.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = a & 0xF
    codes[:, 1::2] = a >> 4
    return codes


def compare_nvfp4(r_bits, w_bits, gc, eps, gs, a_gpu, sf_gpu):
    """Apply the NVFP4 acceptance rule.  Returns (n_exempt, n_codes); raises
    AssertionError on a difference that the rule does not exempt."""
    ref = oracle.rmsnorm_nvfp4(r_bits, w_bits, gc, eps, gs)
    gsf = oracle.f32(gs)
    yn = oracle.bf16_value(ref["yn"])
    u = bf16_ulp(yn)
    M, P = yn.shape
    codes_ref = unpack_codes(ref["a"])
    codes_gpu = unpack_codes(a_gpu)
    e4m3_mids = _e4m3_midpoints()
    exempt = 0
    for m in range(M):
        for b in range(P // 16):
            cols = slice(16 * b, 16 * b + 16)
            sf_r, sf_g = int(ref["a_sf"][m, b]), int(sf_gpu[m, b])
            ynb, ub = yn[m, cols], u[m, cols]
            os_ = ref["os"][m, b]
            cref = codes_ref[m, cols]
            if sf_g != sf_r:
                amax = np.abs(ynb).max()
                ua = bf16_ulp(np.array([amax]))[0]
                lo = np.array([gsf * (amax - ua) / 6.0])
                hi = np.array([gsf * (amax + ua) / 6.0])
                if not _interval_has(e4m3_mids, lo, hi)[0]:
                    raise AssertionError(f"row {m} block {b}: scale {sf_g:#x} != oracle "
                                         f"{sf_r:#x} away from an e4m3 boundary")
                exempt += 1
                cref, _, _, os_ = oracle.nvfp4_block(ynb, gsf, forced_sf=sf_g)
            diff = cref != codes_gpu[m, cols]
            if diff.any():
                a = np.abs(ynb[diff])
                lo = (a - ub[diff]) * os_
                hi = (a + ub[diff]) * os_
                ok = _interval_has(E2M1_MIDPOINTS, lo, hi)
                # the sign bit is never exempt: both sides take it from yn
                ok &= (cref[diff] & 8) == (codes_gpu[m, cols][diff] & 8)
                if not ok.all():
                    j = np.flatnonzero(diff)[np.flatnonzero(~ok)[0]]
                    raise AssertionError(
                        f"row {m} col {16 * b + j}: code {codes_gpu[m, 16 * b + j]:#x} != oracle "
                        f"{cref[j]:#x} (yn {ynb[j]!r}, os {os_!r}) away from an e2m1 boundary")
                exempt += int(diff.sum())
    return exempt, M * P
