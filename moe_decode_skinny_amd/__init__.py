"""moe_decode_skinny_amd: the small-M decode GEMM and its NVFP4 expert-input
epilogue on AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libskinny.so`` (declared in
``include/skinny.h``).  It only marshals arguments: every step runs in the HIP
kernels of the library.  PyTorch provides device memory and streams.  If the
library has not been built this module raises ImportError; there is no
fallback.

Same names as the C ABI:
  skinny_init, skinny_gemm_bf16, skinny_gemm_bf16_noalloc, skinny_gemm_bf16_launch,
  skinny_choose,
  skinny_gemm_unsupported, skinny_launch_unsupported, skinny_gemm_bf16_publish,
  skinny_gemm_bf16_ring,
  skinny_gemm_bf16_ring_launch, skinny_ring_choose, skinny_ring_launch_unsupported,
  skinny_rmsnorm_nvfp4, skinny_rmsnorm_bf16, skinny_dual_norm, skinny_last_error,
  skinny_version
The benchmark's measurement references (a library of their own, not part of
this ABI) are in ``moe_decode_skinny_amd.ceiling``.
Status codes map to exceptions as on the unpooler page (Unpooler.run /
Unpooler.unsupported): EINVAL and EUNSUPPORTED raise ValueError, the others
RuntimeError.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskinny.so")

SKINNY_OK = 0
SKINNY_EINVAL = -1
SKINNY_EUNSUPPORTED = -2
SKINNY_EDEVICE = -3
SKINNY_ELAUNCH = -4
SKINNY_ENOTINIT = -5
SKINNY_PATH_DOT2 = 0
SKINNY_PATH_MFMA = 1
SKINNY_PATH_MFMA_LDS = 2
SKINNY_PATH_MFMA_4X4 = 3
SKINNY_RING_ITEM_MAJOR = 0
SKINNY_RING_XCD_LOCAL = 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python moe_decode_skinny_amd/build.py` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)


class _CLaunch(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("splits", ctypes.c_int), ("waves", ctypes.c_int),
                ("chunks", ctypes.c_int), ("accs", ctypes.c_int), ("rows", ctypes.c_int)]


class Launch(NamedTuple):
    """skinny_launch: path (0 DOT2, 1 MFMA, 2 MFMA_LDS: ring only, 3 MFMA_4X4),
    splits, waves, chunks, accs (MFMA: accumulators; MFMA_4X4: token groups),
    rows."""
    path: int
    splits: int
    waves: int
    chunks: int
    accs: int
    rows: int

    def _c(self) -> _CLaunch:
        return _CLaunch(*self)


class _CMailbox(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stage_state", ctypes.c_void_p),
                ("ticket", ctypes.c_void_p), ("tp", ctypes.c_int), ("rank", ctypes.c_int),
                ("capacity", ctypes.c_int), ("width", ctypes.c_int)]


class _CRingLaunch(ctypes.Structure):
    _fields_ = [("gemm", _CLaunch), ("segment", ctypes.c_int), ("workgroups", ctypes.c_int),
                ("order", ctypes.c_int)]


class RingLaunch(NamedTuple):
    """skinny_ring_launch: gemm (a Launch with splits = 1), segment, workgroups,
    order (SKINNY_RING_ITEM_MAJOR or SKINNY_RING_XCD_LOCAL)."""
    gemm: Launch
    segment: int
    workgroups: int
    order: int = 0

    def _c(self) -> _CRingLaunch:
        return _CRingLaunch(Launch(*self.gemm)._c(), self.segment, self.workgroups, self.order)

    @staticmethod
    def _from_c(c: _CRingLaunch) -> "RingLaunch":
        g = c.gemm
        return RingLaunch(Launch(g.path, g.splits, g.waves, g.chunks, g.accs, g.rows),
                          c.segment, c.workgroups, c.order)


_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sig = {
    "skinny_init": ([_i], _i),
    "skinny_gemm_bf16": ([_vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    "skinny_gemm_bf16_noalloc": ([_vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    "skinny_gemm_bf16_launch": ([_vp, _vp, _vp, _i, _i, _i, ctypes.POINTER(_CLaunch), _vp], _i),
    "skinny_choose": ([_i, _i, _i, _i, ctypes.POINTER(_CLaunch)], _i),
    "skinny_gemm_unsupported": ([_i, _i, _i, _i], _i),
    "skinny_launch_unsupported": ([_i, _i, _i, ctypes.POINTER(_CLaunch)], _i),
    "skinny_gemm_bf16_publish": (
        [_vp, _vp, _vp, _i, _i, _i, ctypes.POINTER(_CLaunch), ctypes.POINTER(_CMailbox), _vp], _i),
    "skinny_gemm_bf16_ring": ([_vp, _vp, _vp, _i, _i, _i, _i, _vp], _i),
    "skinny_gemm_bf16_ring_launch": (
        [_vp, _vp, _vp, _i, _i, _i, _i, ctypes.POINTER(_CRingLaunch), _vp], _i),
    "skinny_ring_choose": ([_i, _i, _i, _i, ctypes.POINTER(_CRingLaunch)], _i),
    "skinny_choose_walk": ([_i, _i, _i, _i, ctypes.POINTER(_CRingLaunch)], _i),
    "skinny_ring_launch_unsupported": ([_i, _i, _i, _i, ctypes.POINTER(_CRingLaunch)], _i),
    "skinny_rmsnorm_nvfp4": ([_vp, _vp, _f, _f, _vp, _vp, _vp, _i, _i, _vp], _i),
    "skinny_rmsnorm_bf16": ([_vp, _vp, _f, _f, _vp, _i, _i, _vp], _i),
    "skinny_dual_norm": ([_vp, _vp, _vp, _f, _f, _vp, _f, _vp, _vp, _f, _f, _vp, _i, _i, _vp], _i),
    "skinny_last_error": ([], ctypes.c_char_p),
    "skinny_version": ([], _i),
}
for _name, (_args, _res) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def skinny_last_error() -> str:
    return _lib.skinny_last_error().decode()


def skinny_version() -> int:
    return _lib.skinny_version()


def _check(status: int) -> None:
    if status == SKINNY_OK:
        return
    msg = skinny_last_error()
    if status in (SKINNY_EINVAL, SKINNY_EUNSUPPORTED):
        raise ValueError(msg)
    raise RuntimeError(f"libskinny status {status}: {msg}")


def _stream(stream, device) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    sdev = getattr(stream, "device", None)
    if sdev is not None and torch.device(sdev) != torch.device(device):
        raise ValueError(f"stream is on {sdev} but the arguments are on {device}")
    return getattr(stream, "cuda_stream", stream)


def _dev_tensor(t, name, dtype):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _common_device(*named):
    """The one device of the (name, tensor) pairs given (None entries skipped);
    ValueError if they are on different devices.  The library runs on the
    current HIP device, so every call is made with this device current."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if dev is None:
            dev, first = t.device, name
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device} but {first} is on {dev}: "
                             "all arguments must be on one device")
    return dev


def _on(device):
    """Context that makes `device` the current device for a library call."""
    import torch

    return torch.cuda.device(device)


def skinny_init(device: int = 0) -> None:
    """Check that `device` is gfx950 and allocate the split-K workspace."""
    _check(_lib.skinny_init(int(device)))


def init(device: int = 0) -> None:
    skinny_init(device)


def skinny_choose(M: int, N: int, K: int, splits: int = 0) -> Launch:
    out = _CLaunch()
    _check(_lib.skinny_choose(M, N, K, splits, ctypes.byref(out)))
    return Launch(out.path, out.splits, out.waves, out.chunks, out.accs, out.rows)


def skinny_gemm_unsupported(M: int, N: int, K: int, splits: int = 0) -> Optional[str]:
    st = _lib.skinny_gemm_unsupported(M, N, K, splits)
    return None if st == SKINNY_OK else skinny_last_error()


def skinny_launch_unsupported(M: int, N: int, K: int, launch: Launch) -> Optional[str]:
    c = Launch(*launch)._c()
    st = _lib.skinny_launch_unsupported(M, N, K, ctypes.byref(c))
    return None if st == SKINNY_OK else skinny_last_error()


def _gemm_args(x, w, y):
    import torch

    xp = _dev_tensor(x, "x", torch.bfloat16)
    wp = _dev_tensor(w, "W", torch.bfloat16)
    yp = _dev_tensor(y, "y", torch.bfloat16)
    if x.dim() != 2 or w.dim() != 2 or y.dim() != 2:
        raise ValueError("x, W and y must be 2-D")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shapes x{tuple(x.shape)} W{tuple(w.shape)} y{tuple(y.shape)}")
    _common_device(("x", x), ("W", w), ("y", y))
    return xp, wp, yp, M, N, K


def skinny_gemm_bf16(x, w, y, splits: int = 0, stream=None):
    """y[M, N] = x[M, K] @ W[N, K]^T into the caller's y; returns y."""
    xp, wp, yp, M, N, K = _gemm_args(x, w, y)
    with _on(x.device):
        _check(_lib.skinny_gemm_bf16(xp, wp, yp, M, N, K, splits, _stream(stream, x.device)))
    return y


def skinny_gemm_bf16_noalloc(x, w, y, splits: int = 0, stream=None):
    """skinny_gemm_bf16 with its split-K partials in the library's static
    scratch array instead of the workspace skinny_init allocated (splits x M
    x N <= 2^18 floats); for callers that cannot allocate.  Calls that overlap
    on one device race on that array.  Returns y."""
    xp, wp, yp, M, N, K = _gemm_args(x, w, y)
    with _on(x.device):
        _check(_lib.skinny_gemm_bf16_noalloc(xp, wp, yp, M, N, K, splits,
                                             _stream(stream, x.device)))
    return y


def skinny_gemm_bf16_launch(x, w, y, launch: Launch, stream=None):
    """The GEMM at an explicit launch shape; returns y."""
    xp, wp, yp, M, N, K = _gemm_args(x, w, y)
    c = Launch(*launch)._c()
    with _on(x.device):
        _check(_lib.skinny_gemm_bf16_launch(xp, wp, yp, M, N, K, ctypes.byref(c),
                                            _stream(stream, x.device)))
    return y


def skinny_gemm_bf16_publish(x, w, y, mailbox, rank: int, stage_state=None, ticket=None,
                             launch: Optional[Launch] = None, stream=None):
    """y = x @ W^T, and y published into mailbox[stage, rank, :M] (bf16
    [3, tp, capacity, N]) with -0.0 stored as +0.0.  The stage comes from
    ticket (int32 [1], stage << 16) if given, else from stage_state (int32
    [2]: [0] the stage, [1] set to it).  Returns y."""
    import torch

    xp, wp, yp, M, N, K = _gemm_args(x, w, y)
    dp = _dev_tensor(mailbox, "mailbox", torch.bfloat16)
    if mailbox.dim() != 4 or mailbox.shape[0] != 3:
        raise ValueError("mailbox must be [3, tp, capacity, width]")
    _, tp, capacity, width = mailbox.shape
    sp = None if stage_state is None else _dev_tensor(stage_state, "stage_state", torch.int32)
    tk = None if ticket is None else _dev_tensor(ticket, "ticket", torch.int32)
    if stage_state is not None and stage_state.numel() != 2:
        raise ValueError("stage_state must be int32 [2]")
    if ticket is not None and ticket.numel() != 1:
        raise ValueError("ticket must be int32 [1]")
    _common_device(("x", x), ("mailbox", mailbox), ("stage_state", stage_state),
                   ("ticket", ticket))
    mb = _CMailbox(dp, sp, tk, tp, int(rank), capacity, width)
    lp = None if launch is None else ctypes.byref(Launch(*launch)._c())
    with _on(x.device):
        _check(_lib.skinny_gemm_bf16_publish(xp, wp, yp, M, N, K, lp, ctypes.byref(mb),
                                             _stream(stream, x.device)))
    return y


def skinny_ring_choose(M: int, N: int, K: int, count: int) -> RingLaunch:
    """The RingLaunch that skinny_gemm_bf16_ring uses."""
    out = _CRingLaunch()
    _check(_lib.skinny_ring_choose(M, N, K, count, ctypes.byref(out)))
    return RingLaunch._from_c(out)


def skinny_choose_walk(M: int, N: int, K: int, splits: int = 0) -> RingLaunch:
    """How skinny_gemm_bf16 runs: segment 0 = the plain kernel at .gemm,
    else the one-item ring launch it is."""
    out = _CRingLaunch()
    _check(_lib.skinny_choose_walk(M, N, K, splits, ctypes.byref(out)))
    return RingLaunch._from_c(out)


def skinny_ring_launch_unsupported(M: int, N: int, K: int, count: int,
                                   launch: RingLaunch) -> Optional[str]:
    c = RingLaunch(*launch)._c()
    st = _lib.skinny_ring_launch_unsupported(M, N, K, count, ctypes.byref(c))
    return None if st == SKINNY_OK else skinny_last_error()


def _ring_args(xs, ws, ys):
    if not (len(xs) == len(ws) == len(ys)) or not xs:
        raise ValueError("xs, ws and ys must be non-empty lists of one length")
    shapes = [_gemm_args(x, w, y) for x, w, y in zip(xs, ws, ys)]
    _common_device(*[(f"xs[{i}]", x) for i, x in enumerate(xs)])
    M, N, K = shapes[0][3:]
    if any(sh[3:] != (M, N, K) for sh in shapes):
        raise ValueError("every ring item must have the same (M, N, K)")
    arr = ctypes.c_void_p * len(xs)
    xa = arr(*[sh[0] for sh in shapes])
    wa = arr(*[sh[1] for sh in shapes])
    ya = arr(*[sh[2] for sh in shapes])
    return xa, wa, ya, len(xs), M, N, K


def skinny_gemm_bf16_ring(xs, ws, ys, stream=None):
    """ys[i] = xs[i] @ ws[i]^T for independent items of one shape, in one
    launch; returns ys."""
    xa, wa, ya, count, M, N, K = _ring_args(xs, ws, ys)
    with _on(xs[0].device):
        _check(_lib.skinny_gemm_bf16_ring(xa, wa, ya, count, M, N, K,
                                          _stream(stream, xs[0].device)))
    return ys


def skinny_gemm_bf16_ring_launch(xs, ws, ys, launch: RingLaunch, stream=None):
    """The ring at an explicit RingLaunch; returns ys."""
    xa, wa, ya, count, M, N, K = _ring_args(xs, ws, ys)
    c = RingLaunch(*launch)._c()
    with _on(xs[0].device):
        _check(_lib.skinny_gemm_bf16_ring_launch(xa, wa, ya, count, M, N, K, ctypes.byref(c),
                                                 _stream(stream, xs[0].device)))
    return ys


def skinny_rmsnorm_nvfp4(r, norm_w, gain_center: float, eps: float, global_scale, a, a_sf,
                         stream=None):
    """NVFP4 expert input of the rows of r into a [M, P/2] u8 and a_sf [M, P/16] u8."""
    import torch

    rp = _dev_tensor(r, "r", torch.bfloat16)
    wp = _dev_tensor(norm_w, "norm_w", torch.bfloat16)
    gp = _dev_tensor(global_scale, "global_scale", torch.float32)
    ap = _dev_tensor(a, "a", torch.uint8)
    sp = _dev_tensor(a_sf, "a_sf", torch.uint8)
    if r.dim() != 2:
        raise ValueError("r must be 2-D")
    M, P = r.shape
    if (tuple(norm_w.shape) != (P,) or global_scale.numel() != 1
            or tuple(a.shape) != (M, P // 2) or tuple(a_sf.shape) != (M, P // 16)):
        raise ValueError("norm_w [P], global_scale [1], a [M, P/2], a_sf [M, P/16]")
    _common_device(("r", r), ("norm_w", norm_w), ("global_scale", global_scale), ("a", a),
                   ("a_sf", a_sf))
    with _on(r.device):
        _check(_lib.skinny_rmsnorm_nvfp4(rp, wp, float(gain_center), float(eps), gp, ap, sp,
                                         M, P, _stream(stream, r.device)))
    return a, a_sf


def skinny_rmsnorm_bf16(r, norm_w, gain_center: float, eps: float, y, stream=None):
    """BF16 edge-layer norm of the rows of r into y [M, P]."""
    import torch

    rp = _dev_tensor(r, "r", torch.bfloat16)
    wp = _dev_tensor(norm_w, "norm_w", torch.bfloat16)
    yp = _dev_tensor(y, "y", torch.bfloat16)
    if r.dim() != 2 or tuple(y.shape) != tuple(r.shape):
        raise ValueError("r and y must be [M, P]")
    M, P = r.shape
    if tuple(norm_w.shape) != (P,):
        raise ValueError("norm_w must be [P]")
    _common_device(("r", r), ("norm_w", norm_w), ("y", y))
    with _on(r.device):
        _check(_lib.skinny_rmsnorm_bf16(rp, wp, float(gain_center), float(eps), yp, M, P,
                                        _stream(stream, r.device)))
    return y


def skinny_dual_norm(partial, residual, post_w, post_gain_center: float, post_eps: float,
                     alpha, beta, next_w, pre_gain_center: float, pre_eps: float, out,
                     stream=None):
    """The dual norm after o_proj: post norm of partial [M, H] (bf16), gated add
    into residual [M, H] (float32, in place), pre norm into out [M, H] (bf16).
    post_w: bf16 [H] or None; alpha: a float or bf16 [H]; beta, next_w: bf16
    [H].  Returns out."""
    import torch

    pp = _dev_tensor(partial, "partial", torch.bfloat16)
    rp = _dev_tensor(residual, "residual", torch.float32)
    op = _dev_tensor(out, "out", torch.bfloat16)
    if partial.dim() != 2 or tuple(residual.shape) != tuple(partial.shape) or \
            tuple(out.shape) != tuple(partial.shape):
        raise ValueError("partial, residual and out must all be [M, H]")
    M, H = partial.shape
    vecs = {}
    for name, t in (("post_w", post_w), ("beta", beta), ("next_w", next_w)):
        if t is None and name == "post_w":
            vecs[name] = None
            continue
        vecs[name] = _dev_tensor(t, name, torch.bfloat16)
        if tuple(t.shape) != (H,):
            raise ValueError(f"{name} must be [H]")
    if isinstance(alpha, torch.Tensor):
        ap, a_s = _dev_tensor(alpha, "alpha", torch.bfloat16), 0.0
        if tuple(alpha.shape) != (H,):
            raise ValueError("alpha must be a float or [H]")
    else:
        ap, a_s = None, float(alpha)
    _common_device(("partial", partial), ("residual", residual), ("out", out),
                   ("post_w", post_w), ("beta", beta), ("next_w", next_w),
                   ("alpha", alpha if isinstance(alpha, torch.Tensor) else None))
    with _on(partial.device):
        _check(_lib.skinny_dual_norm(pp, rp, vecs["post_w"], float(post_gain_center),
                                     float(post_eps), ap, a_s, vecs["beta"], vecs["next_w"],
                                     float(pre_gain_center), float(pre_eps), op, M, H,
                                     _stream(stream, partial.device)))
    return out


__all__ = [
    "Launch", "RingLaunch", "init", "skinny_init", "skinny_gemm_bf16", "skinny_gemm_bf16_launch",
    "skinny_gemm_bf16_noalloc",
    "skinny_choose", "skinny_gemm_unsupported", "skinny_launch_unsupported",
    "skinny_gemm_bf16_publish", "skinny_gemm_bf16_ring", "skinny_gemm_bf16_ring_launch",
    "skinny_ring_choose",
    "skinny_ring_launch_unsupported",
    "skinny_rmsnorm_nvfp4", "skinny_rmsnorm_bf16", "skinny_dual_norm", "skinny_last_error", "skinny_version",
    "LIB_PATH",
]
