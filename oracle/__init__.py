"""Oracle: the plain CPU (binary64) statement of what the GPU library computes.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
(``moe_decode_skinny_amd``) never imports it and shares no code with it.

The arithmetic lives in ``skinny_oracle.c`` (plain C loops, binary64); this
module only marshals numpy arrays into it.  Every bfloat16 array is handled as
its ``uint16`` bit pattern.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against brute force, closed forms, library routines, worked cases and the
format definitions, and ``tests/test_oracle_mutations.py`` checks that
planted mistakes fail those pins.  One function is parity unpinned by the
pages beyond the order of its steps: ``dual_norm`` (the dual norm's formula
and constants are not printed; its pins check the stated reading, given with
its C source).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # Load what is built (build() in __graft_entry__ rebuilds it after a
    # change); compile only when nothing is, never inside a timed run.
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # compiling the checker is not using it

        _build.build()
    _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str):
    """ctypes handle of a compiled oracle with every signature declared (the
    mutation tests load deliberately broken copies this way)."""
    lib = ctypes.CDLL(path)
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_round.argtypes = [ctypes.c_double]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_gemm_bf16.argtypes = [_u16p, _u16p, _u16p] + [ctypes.c_int] * 4
    lib.oracle_gemm_bf16.restype = None
    lib.oracle_gemm_bf16_sampled.argtypes = [
        _u16p, _u16p, ctypes.c_int, _i32p, _i32p, ctypes.c_int, _u16p, ctypes.c_void_p]
    lib.oracle_gemm_bf16_sampled.restype = None
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_nvfp4_block.argtypes = [
        _f64p, ctypes.c_double, ctypes.c_int, _u8p, ctypes.POINTER(ctypes.c_uint8),
        ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_nvfp4_block.restype = None
    lib.oracle_rmsnorm_bf16.argtypes = [
        _u16p, _u16p, ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int, _u16p]
    lib.oracle_rmsnorm_bf16.restype = None
    lib.oracle_rmsnorm_nvfp4.argtypes = [
        _u16p, _u16p, ctypes.c_double, ctypes.c_double, ctypes.c_double,
        ctypes.c_int, ctypes.c_int, _u8p, _u8p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]
    lib.oracle_rmsnorm_nvfp4.restype = None
    lib.oracle_mailbox_publish.argtypes = [
        _u16p, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_mailbox_publish.restype = ctypes.c_int
    lib.oracle_dual_norm.argtypes = [
        _u16p, _f32p, ctypes.c_void_p, ctypes.c_double, ctypes.c_double, ctypes.c_void_p,
        ctypes.c_double, _u16p, _u16p, ctypes.c_double, ctypes.c_double, ctypes.c_int,
        ctypes.c_int, _u16p, ctypes.c_void_p]
    lib.oracle_dual_norm.restype = None
    return lib


class use_library:
    """Context manager: route this module's functions to another compiled
    oracle (a planted-mistake copy) for the duration of the block."""

    def __init__(self, lib):
        self.lib, self.saved = lib, None

    def __enter__(self):
        global _lib
        self.saved, _lib = _lib, self.lib
        return self.lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def f32(v: float) -> float:
    """The binary64 value of ``v`` rounded to binary32: the library takes eps,
    gain_center and global_scale as FP32, so the oracle uses the same
    numbers."""
    return float(np.float32(v))


# ------------------------------------------------------------------ bfloat16
def bf16_value(bits) -> np.ndarray:
    """Values (float64) of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round(values) -> np.ndarray:
    """binary64 -> bfloat16 bits, round to nearest even, one rounding."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.fromiter((lib.oracle_bf16_round(float(t)) for t in flat),
                      dtype=np.uint16, count=flat.size)
    return out.reshape(v.shape)


# ---------------------------------------------------------------------- GEMM
def gemm_bf16(x_bits: np.ndarray, w_bits: np.ndarray, threads: int = 1) -> np.ndarray:
    """y = bf16(x @ W^T) with a binary64 sum over k ascending.

    x_bits [M, K] and w_bits [N, K] are bfloat16 bit patterns; returns y bits
    [M, N]."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError(f"K mismatch {K} != {K2}")
    y = np.empty((M, N), dtype=np.uint16)
    lib.oracle_gemm_bf16(x, w, y, M, N, K, int(threads))
    return y


def gemm_bf16_sampled(x_bits, w_bits, rows, cols):
    """The oracle GEMM at positions (rows[i], cols[i]) only.

    Returns (y bits [count], exact binary64 sums [count])."""
    lib = _load()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    r = np.ascontiguousarray(rows, dtype=np.int32)
    c = np.ascontiguousarray(cols, dtype=np.int32)
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    if r.size and (r.min() < 0 or r.max() >= x.shape[0] or c.min() < 0 or c.max() >= w.shape[0]):
        raise ValueError("sample position out of range")
    out = np.empty(r.size, dtype=np.uint16)
    exact = np.empty(r.size, dtype=np.float64)
    lib.oracle_gemm_bf16_sampled(x, w, x.shape[1], r, c, r.size, out, _ptr(exact))
    return out, exact


# -------------------------------------------------------------------- codecs
def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e2m1_encode(v: float) -> int:
    return int(_load().oracle_e2m1_encode(float(v)))


def nvfp4_block(yn16, global_scale: float, forced_sf: int = -1):
    """Quantize one 16-value block; returns (codes[16], sf, pre[16], os)."""
    lib = _load()
    yn = np.ascontiguousarray(yn16, dtype=np.float64)
    if yn.shape != (16,):
        raise ValueError("a block has 16 values")
    codes = np.empty(16, dtype=np.uint8)
    sf = ctypes.c_uint8(0)
    pre = np.empty(16, dtype=np.float64)
    os_ = ctypes.c_double(0.0)
    lib.oracle_nvfp4_block(yn, float(global_scale), int(forced_sf), codes,
                           ctypes.byref(sf), _ptr(pre), ctypes.addressof(os_))
    return codes, int(sf.value), pre, float(os_.value)


# ---------------------------------------------------------------------- norm
def rmsnorm_bf16(r_bits, w_bits, gain_center: float, eps: float) -> np.ndarray:
    """yn = bf16(r / sqrt(mean(r^2) + eps) * (w + gain_center)), per row.

    gain_center and eps are taken as the FP32 numbers the library receives."""
    lib = _load()
    r = np.ascontiguousarray(r_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    M, P = r.shape
    if w.shape != (P,):
        raise ValueError("norm weight must be [P]")
    yn = np.empty((M, P), dtype=np.uint16)
    lib.oracle_rmsnorm_bf16(r, w, f32(gain_center), f32(eps), M, P, yn)
    return yn


def rmsnorm_nvfp4(r_bits, w_bits, gain_center: float, eps: float, global_scale: float):
    """The NVFP4 expert input.  Returns a dict with
    a [M, P/2] u8, a_sf [M, P/16] u8, yn [M, P] bf16 bits, pre [M, P] f64 (the
    scaled value before e2m1 rounding) and os [M, P/16] f64 (output scales)."""
    lib = _load()
    r = np.ascontiguousarray(r_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    M, P = r.shape
    if w.shape != (P,) or P % 16:
        raise ValueError("need norm weight [P] and P % 16 == 0")
    a = np.empty((M, P // 2), dtype=np.uint8)
    a_sf = np.empty((M, P // 16), dtype=np.uint8)
    yn = np.empty((M, P), dtype=np.uint16)
    pre = np.empty((M, P), dtype=np.float64)
    osc = np.empty((M, P // 16), dtype=np.float64)
    lib.oracle_rmsnorm_nvfp4(r, w, f32(gain_center), f32(eps), f32(global_scale),
                             M, P, a, a_sf, _ptr(yn), _ptr(pre), _ptr(osc))
    return {"a": a, "a_sf": a_sf, "yn": yn, "pre": pre, "os": osc}


# ------------------------------------------------------------------- publish
def mailbox_publish(y_bits, mailbox, rank: int, stage_state=None, ticket=None):
    """The zero-copy publish of y [M, width] into this rank's slot of
    mailbox [3, tp, capacity, width] (uint16 bf16 bits, updated in place).
    With a ticket (int32 [1]) the stage comes from it and stage_state, if
    given, is not used; otherwise stage_state (int32 [2]) gives the stage and
    is updated in place.  Returns the stage used, or -1 if it was outside
    0..2 (nothing written)."""
    lib = _load()
    y = np.ascontiguousarray(y_bits, dtype=np.uint16)
    if mailbox.dtype != np.uint16 or mailbox.ndim != 4 or not mailbox.flags.c_contiguous:
        raise ValueError("mailbox must be a contiguous uint16 [3, tp, capacity, width] array")
    stages, tp, capacity, width = mailbox.shape
    M = y.shape[0]
    if stages != 3 or y.shape != (M, width) or M > capacity or not 0 <= rank < tp:
        raise ValueError("shapes do not fit the mailbox")
    if stage_state is None and ticket is None:
        raise ValueError("give stage_state or ticket")
    st = None if stage_state is None else stage_state
    tk = None if ticket is None else np.ascontiguousarray(ticket, dtype=np.int32)
    if st is not None and (st.dtype != np.int32 or st.shape != (2,) or not st.flags.c_contiguous):
        raise ValueError("stage_state must be a contiguous int32 [2] array")
    return lib.oracle_mailbox_publish(y, M, width, mailbox, tp, rank, capacity, _ptr(st), _ptr(tk))


# ----------------------------------------------------------------- dual norm
def dual_norm(partial_bits, stream, post_w_bits, post_gc: float, post_eps: float, alpha,
              beta_bits, next_w_bits, pre_gc: float, pre_eps: float):
    """The single-GPU dual norm after o_proj (a reading: see the C source).

    partial bf16 bits [M, H]; stream float32 [M, H] (a new updated array is
    returned, the input is not modified); post_w bf16 bits [H] or None;
    alpha a float (scalar) or bf16 bits [H]; beta, next_w bf16 bits [H].
    The FP32 scalars are taken as the FP32 numbers the library receives.
    Returns (out bf16 bits [M, H], updated stream float32 [M, H], h bf16 bits)."""
    lib = _load()
    p = np.ascontiguousarray(partial_bits, dtype=np.uint16)
    M, H = p.shape
    st = np.array(stream, dtype=np.float32, copy=True, order="C")
    if st.shape != (M, H):
        raise ValueError("stream must be [M, H]")
    pw = None if post_w_bits is None else np.ascontiguousarray(post_w_bits, dtype=np.uint16)
    if np.isscalar(alpha):
        al, a_s = None, f32(float(alpha))
    else:
        al, a_s = np.ascontiguousarray(alpha, dtype=np.uint16), 0.0
    be = np.ascontiguousarray(beta_bits, dtype=np.uint16)
    nw = np.ascontiguousarray(next_w_bits, dtype=np.uint16)
    for name, v in (("post_w", pw), ("alpha", al), ("beta", be), ("next_w", nw)):
        if v is not None and v.shape != (H,):
            raise ValueError(f"{name} must be [H]")
    out = np.empty((M, H), dtype=np.uint16)
    h = np.empty((M, H), dtype=np.uint16)
    lib.oracle_dual_norm(p, st, _ptr(pw), f32(post_gc), f32(post_eps), _ptr(al), a_s, be, nw,
                         f32(pre_gc), f32(pre_eps), M, H, out, _ptr(h))
    return out, st, h
