"""Python binding of ``libswiglu_probs.so`` (C ABI in ``include/swiglu_probs.h``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are handed to
the C functions of the same names. Every step of the activation runs in the HIP
kernels; there is no CPU or PyTorch fallback, and a missing library is an error.

bf16 tensors may be given as ``torch.bfloat16`` or as ``torch.int16``/``uint16``
views of the bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

from . import build as _build

SWIGLU_OK = 0
SWIGLU_ERR_INVALID_ARG = 1
SWIGLU_ERR_ALIGNMENT = 2
SWIGLU_ERR_HIP = 3

_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "swiglu_probs_fwd": [_vp, _vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp, ctypes.c_int, _vp],
    "swiglu_probs_bwd": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp,
                         ctypes.c_int, _vp],
    "swiglu_probs_fwd_ex": [_vp, _vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp, ctypes.c_int,
                            _vp, ctypes.c_int],
    "swiglu_probs_bwd_ex": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp,
                            ctypes.c_int, _vp, ctypes.c_int],
    "swiglu_probs_fwd_timed": [_vp, _vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp, ctypes.c_int,
                               _vp, ctypes.c_int, _vp, _vp],
    "swiglu_probs_bwd_timed": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_float, _vp, _vp,
                               ctypes.c_int, _vp, ctypes.c_int, _vp, _vp],
    "swiglu_probs_default_workgroups": [ctypes.c_int, _i64, _i64],
    "swiglu_probs_status_string": [ctypes.c_int],
    "swiglu_probs_last_hip_error": [],
    "swiglu_probs_abi_version": [],
}
_RESTYPES = {"swiglu_probs_status_string": ctypes.c_char_p}


class SwigluProbsError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} failed: {status_string(status)} (status {status}"
        if status == SWIGLU_ERR_HIP:
            msg += f", hipError {hip_error}"
        super().__init__(msg + ")")


def library_path() -> str:
    return _build.lib_path("swiglu_probs")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (building it first if nothing is built) the HIP library; cached."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or library_path()
        if not os.path.exists(p):
            _build.build_lib("swiglu_probs")
        lib = ctypes.CDLL(p)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, ctypes.c_int)
        if lib.swiglu_probs_abi_version() != 1:
            raise RuntimeError("libswiglu_probs.so ABI version mismatch")
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().swiglu_probs_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != SWIGLU_OK:
        raise SwigluProbsError(fn, status, load_library().swiglu_probs_last_hip_error())


def _bf16_2d(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bf16 (or its int16/uint16 bits), got {t.dtype}")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")
    return t


def _on_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must live on one device")
    return dev


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _row_meta(rows, probs, n_used, permutation_map):
    if probs.dtype != torch.float32 or probs.numel() != rows or not probs.is_contiguous():
        raise ValueError("probs must be contiguous fp32 with one value per row ([rows] or [rows, 1])")
    if n_used is not None and (n_used.dtype != torch.int32 or n_used.numel() != 1):
        raise ValueError("n_used must be a device int32 scalar tensor")
    if permutation_map is not None and (permutation_map.dtype != torch.int32 or
                                        permutation_map.numel() != rows or
                                        not permutation_map.is_contiguous()):
        raise ValueError("permutation_map must be contiguous int32 [rows]")


def swiglu_probs_fwd(x: torch.Tensor, probs: torch.Tensor, y: torch.Tensor, limit: float, *,
                     n_used: Optional[torch.Tensor] = None,
                     permutation_map: Optional[torch.Tensor] = None, zero_padding: bool = False,
                     stream=None, num_workgroups: int = 0, events=None) -> torch.Tensor:
    """y = bf16(silu(clamp(gate, max=limit)) * clamp(up, -limit, limit) * probs), in place into ``y``.

    ``events``: optional (start, stop) HIP event handles (ints) that record the kernel's own
    start and end (swiglu_probs_fwd_timed); for benchmarks."""
    _bf16_2d(x, "x")
    _bf16_2d(y, "y")
    rows, two_inter = x.shape
    if two_inter % 2 or y.shape != (rows, two_inter // 2):
        raise ValueError("x must be [rows, 2*inter] and y [rows, inter]")
    _row_meta(rows, probs, n_used, permutation_map)
    dev = _on_device(x, probs, y, n_used, permutation_map)
    lib = load_library()
    args = (_ptr(x), _ptr(probs), _ptr(y), rows, two_inter // 2, float(limit), _ptr(n_used),
            _ptr(permutation_map), int(bool(zero_padding)), _stream(stream, dev), int(num_workgroups))
    if events is None:
        st = lib.swiglu_probs_fwd_ex(*args)
    else:
        st = lib.swiglu_probs_fwd_timed(*args, events[0], events[1])
    _check("swiglu_probs_fwd", st)
    return y


def swiglu_probs_bwd(x: torch.Tensor, probs: torch.Tensor, grad_y: torch.Tensor,
                     grad_x: torch.Tensor, grad_probs: Optional[torch.Tensor], limit: float, *,
                     n_used: Optional[torch.Tensor] = None,
                     permutation_map: Optional[torch.Tensor] = None, zero_padding: bool = False,
                     stream=None, num_workgroups: int = 0, events=None):
    """d_gate / d_up into the halves of ``grad_x``; per-slot probability gradient into ``grad_probs``.

    ``events``: as for swiglu_probs_fwd (swiglu_probs_bwd_timed)."""
    _bf16_2d(x, "x")
    _bf16_2d(grad_y, "grad_y")
    _bf16_2d(grad_x, "grad_x")
    rows, two_inter = x.shape
    if two_inter % 2 or grad_y.shape != (rows, two_inter // 2) or grad_x.shape != x.shape:
        raise ValueError("x, grad_x must be [rows, 2*inter] and grad_y [rows, inter]")
    _row_meta(rows, probs, n_used, permutation_map)
    if grad_probs is not None and (grad_probs.dtype != torch.float32 or grad_probs.numel() != rows
                                   or not grad_probs.is_contiguous()):
        raise ValueError("grad_probs must be contiguous fp32 with one value per row")
    dev = _on_device(x, probs, grad_y, grad_x, grad_probs, n_used, permutation_map)
    lib = load_library()
    args = (_ptr(x), _ptr(probs), _ptr(grad_y), _ptr(grad_x), _ptr(grad_probs), rows, two_inter // 2,
            float(limit), _ptr(n_used), _ptr(permutation_map), int(bool(zero_padding)),
            _stream(stream, dev), int(num_workgroups))
    if events is None:
        st = lib.swiglu_probs_bwd_ex(*args)
    else:
        st = lib.swiglu_probs_bwd_timed(*args, events[0], events[1])
    _check("swiglu_probs_bwd", st)
    return grad_x, grad_probs


def swiglu_probs_default_workgroups(direction: str, rows: int, inter: int) -> int:
    d = {"fwd": 0, "bwd": 1}[direction]
    return int(load_library().swiglu_probs_default_workgroups(d, rows, inter))


# -- allocating conveniences and an autograd Function -------------------------
def _new_output(shape, like: torch.Tensor, kw) -> torch.Tensor:
    """An output the kernels write in full: rows that are not live (past n_used, or
    dummy map entries) are written only with zero_padding, so otherwise they start as
    zeros here rather than as whatever the allocation held."""
    partial = (kw.get("n_used") is not None or kw.get("permutation_map") is not None) \
        and not kw.get("zero_padding", False)
    return (torch.zeros if partial else torch.empty)(shape, dtype=like.dtype, device=like.device)


def forward(x: torch.Tensor, probs: torch.Tensor, limit: float, **kw) -> torch.Tensor:
    y = _new_output((x.shape[0], x.shape[1] // 2), x, kw)
    return swiglu_probs_fwd(x, probs, y, limit, **kw)


def backward(x: torch.Tensor, probs: torch.Tensor, grad_y: torch.Tensor, limit: float, **kw):
    """(grad_x, grad_probs). grad_probs slots that no live row maps to are never written
    by the kernel, so they start (and stay) zero: no probability gradient flows there."""
    grad_x = _new_output(tuple(x.shape), x, kw)
    grad_probs = torch.zeros(probs.shape, dtype=torch.float32, device=x.device)
    return swiglu_probs_bwd(x, probs, grad_y, grad_x, grad_probs, limit, **kw)


class SwigluProbs(torch.autograd.Function):
    """silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs with the HIP kernels.

    Saves only ``x`` and ``probs``; the backward recomputes the activation.
    ``x`` bf16 [rows, 2*inter] contiguous, ``probs`` fp32 [rows, 1] or [rows].
    """

    @staticmethod
    def forward(ctx, x, probs, limit):
        ctx.save_for_backward(x, probs)
        ctx.limit = float(limit)
        return forward(x, probs, limit)

    @staticmethod
    def backward(ctx, grad_y):
        x, probs = ctx.saved_tensors
        grad_x, grad_probs = backward(x, probs, grad_y.contiguous(), ctx.limit)
        return grad_x, grad_probs.view(probs.shape), None
