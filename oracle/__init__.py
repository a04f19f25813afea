"""CPU oracle for the clamped SwiGLU x probs expert activation (forward and backward).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP library and never imports it; both sides only share the seeded
input generators, which hold none of the method's arithmetic.

The arithmetic lives in ``swiglu_oracle.c`` (plain C loops, compiled with gcc
without fast-math or FMA contraction); this module is ctypes marshalling of
numpy arrays. Sources, per function:

* ``fwd`` / ``bwd``: NeMo AutoModel "moe/swiglu_triton" page (module docstring:
  the formula, fp32 math, one rounding, d_gate/d_up into the halves of grad_x,
  per-row probability gradient; inclusive clamp masks as torch.clamp), and the
  Megatron-Core "core.inference.moe.batch_invariant" page (_swiglu_with_probs_kernel
  and swiglu_with_probs: permutation_map, n_used, zero_padding;
  _weighted_silu_mul_bounded_kernel: rows past the device bound are neither read
  nor written).
* ``fwd_f64`` / ``bwd_f64``: the same formula in fp64 with no rounding; used by the
  finite-difference and brute-force pins.
* ``bf16_rne``: fp32 -> bf16, round to nearest even (the single final rounding).

Pinning: every function here is checked by ``tests/test_oracle_pins.py`` against
values fixed independently of it (torch library routines, fp64 autograd, central
finite differences, closed forms, brute force, structural invariants). The pins
live in ``tests/oracle_pins.py``, whose module docstring maps each part of the
oracle to the pin that checks it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)


def host_cores() -> int:
    """Cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def default_threads() -> int:
    """Host threads the oracle uses: every core this process may run on, capped by
    OMP_NUM_THREADS when that is set (a host shared between GPUs sets it to each GPU's
    share of the cores), and by the library's limit of 256."""
    n = host_cores()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, min(256, n))


def _ptr(a: Optional[np.ndarray], ptype):
    if a is None:
        return None
    return a.ctypes.data_as(ptype)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    if a.dtype != dtype:
        raise TypeError(f"expected dtype {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


class Oracle:
    """ctypes view of one build of ``swiglu_oracle.c``.

    ``lib_path`` defaults to the in-tree build and is compiled on first use if it
    is missing. Tests that plant a mistake in a copy of the C source load that
    copy through this same class.
    """

    def __init__(self, lib_path: Optional[str] = None):
        if lib_path is None:
            lib_path = _build.LIB_PATH
            if not os.path.exists(lib_path):
                _build.build()
        self.lib_path = lib_path
        lib = ctypes.CDLL(lib_path)
        lib.oracle_bf16_rne_array.argtypes = [_f32p, _u16p, ctypes.c_int64]
        lib.oracle_bf16_rne_array.restype = None
        lib.oracle_swiglu_fwd.argtypes = [_u16p, _f32p, _u16p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_float, _i32p, _i32p, ctypes.c_int, ctypes.c_int]
        lib.oracle_swiglu_fwd.restype = ctypes.c_int
        lib.oracle_swiglu_bwd.argtypes = [_u16p, _f32p, _u16p, _u16p, _f32p, _f64p, _f64p,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                          _i32p, _i32p, ctypes.c_int, ctypes.c_int]
        lib.oracle_swiglu_bwd.restype = ctypes.c_int
        lib.oracle_swiglu_fwd_f64.argtypes = [_f64p, _f64p, _f64p, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_double]
        lib.oracle_swiglu_fwd_f64.restype = ctypes.c_int
        lib.oracle_swiglu_bwd_f64.argtypes = [_f64p, _f64p, _f64p, _f64p, _f64p,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
        lib.oracle_swiglu_bwd_f64.restype = ctypes.c_int
        self.lib = lib

    # -- fp32 -> bf16 ------------------------------------------------------
    def bf16_rne(self, f: np.ndarray) -> np.ndarray:
        f = _c(np.asarray(f), np.float32)
        out = np.empty(f.shape, dtype=np.uint16)
        self.lib.oracle_bf16_rne_array(_ptr(f, _f32p), _ptr(out, _u16p), f.size)
        return out

    # -- forward ---------------------------------------------------------
    def fwd(self, x: np.ndarray, probs: np.ndarray, limit: float, *,
            n_used: Optional[int] = None, permutation_map: Optional[np.ndarray] = None,
            zero_padding: bool = False, out: Optional[np.ndarray] = None,
            threads: Optional[int] = None) -> np.ndarray:
        """y[rows, inter] (bf16 bits) from x[rows, 2*inter] (bf16 bits) and probs[rows] fp32.

        ``out`` supplies the initial content of y (rows that are not live and not
        zero-padded keep it); by default it is a fresh array filled with 0xFFFF.
        """
        x = _c(x, np.uint16)
        rows, two_inter = x.shape
        inter = two_inter // 2
        probs = _c(np.asarray(probs).reshape(-1), np.float32)
        if probs.shape[0] != rows:
            raise ValueError("probs must hold one value per row")
        y = np.full((rows, inter), 0xFFFF, dtype=np.uint16) if out is None else _c(out, np.uint16)
        nu = None if n_used is None else np.array([n_used], dtype=np.int32)
        pm = None if permutation_map is None else _c(permutation_map, np.int32)
        rc = self.lib.oracle_swiglu_fwd(_ptr(x, _u16p), _ptr(probs, _f32p), _ptr(y, _u16p),
                                        rows, inter, float(limit), _ptr(nu, _i32p), _ptr(pm, _i32p),
                                        int(bool(zero_padding)), threads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_swiglu_fwd rejected its arguments (rc={rc})")
        return y

    # -- backward ----------------------------------------------------------
    def bwd(self, x: np.ndarray, probs: np.ndarray, grad_y: np.ndarray, limit: float, *,
            n_used: Optional[int] = None, permutation_map: Optional[np.ndarray] = None,
            zero_padding: bool = False, grad_x_out: Optional[np.ndarray] = None,
            grad_probs_out: Optional[np.ndarray] = None,
            threads: Optional[int] = None) -> dict:
        """Returns ``grad_x`` (bf16 bits [rows, 2*inter]), ``grad_probs`` (fp32 [rows]),
        ``grad_probs_f64`` (the fp64 row sums) and ``row_scale`` (sum of |terms| per slot).

        Slots that no live row maps to keep their initial content: ``grad_probs_out``
        (default: NaN-filled) and NaN for the fp64 arrays.
        """
        x = _c(x, np.uint16)
        rows, two_inter = x.shape
        inter = two_inter // 2
        probs = _c(np.asarray(probs).reshape(-1), np.float32)
        grad_y = _c(grad_y, np.uint16)
        if grad_y.shape != (rows, inter) or probs.shape[0] != rows:
            raise ValueError("shape mismatch")
        gx = (np.full((rows, 2 * inter), 0xFFFF, dtype=np.uint16) if grad_x_out is None
              else _c(grad_x_out, np.uint16))
        gp = (np.full(rows, np.nan, dtype=np.float32) if grad_probs_out is None
              else _c(grad_probs_out, np.float32))
        gp64 = np.full(rows, np.nan, dtype=np.float64)
        scale = np.full(rows, np.nan, dtype=np.float64)
        nu = None if n_used is None else np.array([n_used], dtype=np.int32)
        pm = None if permutation_map is None else _c(permutation_map, np.int32)
        rc = self.lib.oracle_swiglu_bwd(_ptr(x, _u16p), _ptr(probs, _f32p), _ptr(grad_y, _u16p),
                                        _ptr(gx, _u16p), _ptr(gp, _f32p), _ptr(gp64, _f64p),
                                        _ptr(scale, _f64p), rows, inter, float(limit),
                                        _ptr(nu, _i32p), _ptr(pm, _i32p), int(bool(zero_padding)),
                                        threads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_swiglu_bwd rejected its arguments (rc={rc})")
        return {"grad_x": gx, "grad_probs": gp, "grad_probs_f64": gp64, "row_scale": scale}

    # -- fp64, no rounding -------------------------------------------------
    def fwd_f64(self, x: np.ndarray, probs: np.ndarray, limit: float) -> np.ndarray:
        x = _c(x, np.float64)
        rows, two_inter = x.shape
        probs = _c(np.asarray(probs, dtype=np.float64).reshape(-1), np.float64)
        y = np.empty((rows, two_inter // 2), dtype=np.float64)
        rc = self.lib.oracle_swiglu_fwd_f64(_ptr(x, _f64p), _ptr(probs, _f64p), _ptr(y, _f64p),
                                            rows, two_inter // 2, float(limit))
        if rc != 0:
            raise ValueError("oracle_swiglu_fwd_f64 rejected its arguments")
        return y

    def bwd_f64(self, x: np.ndarray, probs: np.ndarray, grad_y: np.ndarray, limit: float):
        x = _c(x, np.float64)
        rows, two_inter = x.shape
        probs = _c(np.asarray(probs, dtype=np.float64).reshape(-1), np.float64)
        grad_y = _c(grad_y, np.float64)
        gx = np.empty_like(x)
        gp = np.empty(rows, dtype=np.float64)
        rc = self.lib.oracle_swiglu_bwd_f64(_ptr(x, _f64p), _ptr(probs, _f64p), _ptr(grad_y, _f64p),
                                            _ptr(gx, _f64p), _ptr(gp, _f64p), rows, two_inter // 2,
                                            float(limit))
        if rc != 0:
            raise ValueError("oracle_swiglu_bwd_f64 rejected its arguments")
        return gx, gp


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from the in-tree source (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
