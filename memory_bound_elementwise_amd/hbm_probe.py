"""Binding of ``libhbm_probe.so`` (``include/hbm_probe.h``): plain streaming kernels
that measure the practical HBM ceiling (mixed read:write streams and the one-way
read-only and write-only ends) and calibrate the byte counters."""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

_lib = None


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        p = _build.lib_path("hbm_probe")
        if not os.path.exists(p):
            _build.build_lib("hbm_probe")
        lib = ctypes.CDLL(p)
        lib.hbm_probe_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        lib.hbm_probe_stream.restype = ctypes.c_int
        lib.hbm_probe_read.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.hbm_probe_read.restype = ctypes.c_int
        lib.hbm_probe_fill.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
        lib.hbm_probe_fill.restype = ctypes.c_int
        _lib = lib
    return _lib


def hbm_probe_stream(srcs, dsts, num_workgroups: int = 0, stream=None) -> None:
    """dst[i] = XOR of srcs at i, for each dst; all tensors same byte size, multiple of 16."""
    nbytes = srcs[0].numel() * srcs[0].element_size()
    for t in list(srcs) + list(dsts):
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("probe tensors must be contiguous GPU tensors of one byte size")
    if nbytes % 16:
        raise ValueError("byte size must be a multiple of 16")
    s = (ctypes.c_void_p * len(srcs))(*[t.data_ptr() for t in srcs])
    d = (ctypes.c_void_p * len(dsts))(*[t.data_ptr() for t in dsts])
    st = torch.cuda.current_stream(srcs[0].device).cuda_stream if stream is None else stream
    rc = load_library().hbm_probe_stream(s, len(srcs), d, len(dsts), nbytes // 16,
                                         int(num_workgroups), st)
    if rc != 0:
        raise RuntimeError(f"hbm_probe_stream failed with code {rc}")


def _byte_size(tensors) -> int:
    nbytes = tensors[0].numel() * tensors[0].element_size()
    for t in tensors:
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("probe tensors must be contiguous GPU tensors of one byte size")
    if nbytes % 16:
        raise ValueError("byte size must be a multiple of 16")
    return nbytes


def hbm_probe_read(srcs, key: int, sink, num_workgroups: int = 0, stream=None) -> None:
    """Read every source once; `sink` (16 bytes on the device) is written only by lanes
    whose XOR of what they read equals `key` in all four words."""
    nbytes = _byte_size(srcs)
    if sink.numel() * sink.element_size() < 16 or sink.device.type != "cuda":
        raise ValueError("sink must be a GPU tensor of at least 16 bytes")
    s = (ctypes.c_void_p * len(srcs))(*[t.data_ptr() for t in srcs])
    st = torch.cuda.current_stream(srcs[0].device).cuda_stream if stream is None else stream
    rc = load_library().hbm_probe_read(s, len(srcs), nbytes // 16, int(key) & 0xFFFFFFFF, sink.data_ptr(),
                                       int(num_workgroups), st)
    if rc != 0:
        raise RuntimeError(f"hbm_probe_read failed with code {rc}")


def hbm_probe_fill(dsts, value: int, num_workgroups: int = 0, stream=None) -> None:
    """Write `value` to every 32-bit word of each destination, reading nothing."""
    nbytes = _byte_size(dsts)
    d = (ctypes.c_void_p * len(dsts))(*[t.data_ptr() for t in dsts])
    st = torch.cuda.current_stream(dsts[0].device).cuda_stream if stream is None else stream
    rc = load_library().hbm_probe_fill(d, len(dsts), nbytes // 16, int(value) & 0xFFFFFFFF,
                                       int(num_workgroups), st)
    if rc != 0:
        raise RuntimeError(f"hbm_probe_fill failed with code {rc}")
