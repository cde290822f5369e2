"""Binding of libskinny_ceiling.so (include/skinny_ceiling.h): the benchmark's
measurement references, a library of their own beside libskinny.  Not steps
of the method: one empty launch, one launch that streams a buffer the way
the GEMM kernels stream weights (unpooler page, module description: a decode
GEMM call is one pass over its weight), and that stream ended as a GEMM
workgroup ends (a cross-wave combine through LDS, then a store).  Argument marshalling only; raises
ImportError when the library is not built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

from . import _dev_tensor, _common_device, _on, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskinny_ceiling.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python moe_decode_skinny_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i = ctypes.c_void_p, ctypes.c_int
_lib.skinny_ceiling_empty.argtypes = [_vp]
_lib.skinny_ceiling_empty.restype = _i
_lib.skinny_ceiling_stream.argtypes = [_vp, ctypes.c_longlong, _vp, _i, _vp]
_lib.skinny_ceiling_stream.restype = _i
_lib.skinny_ceiling_stream_store.argtypes = [_vp, ctypes.c_longlong, _vp, _i, _vp]
_lib.skinny_ceiling_stream_store.restype = _i
_lib.skinny_ceiling_last_error.argtypes = []
_lib.skinny_ceiling_last_error.restype = ctypes.c_char_p


def skinny_ceiling_last_error() -> str:
    return _lib.skinny_ceiling_last_error().decode()


def _check(status: int) -> None:
    if status == 0:
        return
    msg = skinny_ceiling_last_error()
    if status == -1:
        raise ValueError(msg)
    raise RuntimeError(f"libskinny_ceiling status {status}: {msg}")


def skinny_ceiling_empty(device=0, stream=None) -> None:
    """One launch of an empty kernel."""
    import torch

    dev = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
    with _on(dev):
        _check(_lib.skinny_ceiling_empty(_stream(stream, dev)))


def skinny_ceiling_stream(src, sink, loads_per_lane: int = 4, stream=None) -> None:
    """One launch that streams the bytes of src (a contiguous device tensor) as
    the GEMM kernels stream weights; sink is int32 [src bytes / (8192 *
    loads_per_lane)] (include/skinny_ceiling.h)."""
    import torch

    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    kp = _dev_tensor(sink, "sink", torch.int32)
    nbytes = src.numel() * src.element_size()
    if loads_per_lane in (1, 2, 4, 8) and sink.numel() * 8192 * loads_per_lane != nbytes:
        raise ValueError("sink must hold one word per 8192 * loads_per_lane bytes of src")
    _common_device(("src", src), ("sink", sink))
    with _on(src.device):
        _check(_lib.skinny_ceiling_stream(src.data_ptr(), nbytes, kp, int(loads_per_lane),
                                          _stream(stream, src.device)))


def skinny_ceiling_stream_store(src, out, loads_per_lane: int = 1, stream=None) -> None:
    """The loads of skinny_ceiling_stream, then 64 words per workgroup combined
    across its waves through LDS and stored; out is int32 [64 * src bytes /
    (8192 * loads_per_lane)] (include/skinny_ceiling.h)."""
    import torch

    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    op = _dev_tensor(out, "out", torch.int32)
    nbytes = src.numel() * src.element_size()
    if loads_per_lane in (1, 2, 4, 8) and out.numel() * 8192 * loads_per_lane != 64 * nbytes:
        raise ValueError("out must hold 64 words per 8192 * loads_per_lane bytes of src")
    _common_device(("src", src), ("out", out))
    with _on(src.device):
        _check(_lib.skinny_ceiling_stream_store(src.data_ptr(), nbytes, op, int(loads_per_lane),
                                                _stream(stream, src.device)))


__all__ = ["skinny_ceiling_empty", "skinny_ceiling_stream", "skinny_ceiling_stream_store",
           "skinny_ceiling_last_error", "LIB_PATH"]
