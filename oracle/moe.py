"""CPU oracle for the MoE elementwise operations next to the activation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). ctypes marshalling of
numpy arrays around ``moe_oracle.c``; the arithmetic and its sources are in that
file's header:

* ``residual_add``       Megatron-Core "core.fusions.fused_moe_residual_add" page
* ``router_weight_fwd``,
  ``router_weight_bwd``  NeMo AutoModel "moe/optimized_ops" page (_RouterWeightMulFunction)
* ``squared_relu_probs`` Megatron-Core "core.inference.moe.batch_invariant" page
                         (_squared_relu_with_probs_kernel, squared_relu_with_probs)
* ``squared_relu_probs_bwd`` the chain rule through that forward (the page gives none)
* ``unpermute``          same page (_unpermute_tokens_in_expert_order_kernel)

Element types are "bf16", "f16" or "f32"; 16-bit arrays are uint16 bit patterns. Every
call takes ``threads`` (default: ``oracle.default_threads()``); the bits do not depend on it.
Pins: ``tests/moe_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build
from . import default_threads

DTYPES = {"bf16": 0, "f16": 1, "f32": 2}
NP = {"bf16": np.uint16, "f16": np.uint16, "f32": np.float32}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dt):
        raise TypeError(f"expected {np.dtype(dt)}, got {a.dtype}")
    return a


class MoeOracle:
    def __init__(self, lib_path: Optional[str] = None):
        if lib_path is None:
            lib_path = _build.MOE_LIB_PATH
            if not os.path.exists(lib_path):
                _build.compile_oracle(_build.MOE_SOURCE, _build.MOE_LIB_PATH)
        lib = ctypes.CDLL(lib_path)
        lib.oracle_f16_from_f32.argtypes = [_vp, _vp, _i64]
        lib.oracle_f32_from_f16.argtypes = [_vp, _vp, _i64]
        _int = ctypes.c_int
        lib.oracle_residual_add.argtypes = [_vp, _vp, _vp, _vp, _i64, _int, _int]
        lib.oracle_router_weight_fwd.argtypes = [_vp, _int, _vp, _vp, _int, _i64, _i64, _int]
        lib.oracle_router_weight_bwd.argtypes = [_vp, _int, _vp, _int, _vp, _vp, _vp, _vp, _vp, _i64,
                                                 _i64, _int]
        lib.oracle_squared_relu_probs_fwd.argtypes = [_vp, _vp, _vp, _i64, _i64, _int, ctypes.c_float,
                                                      _vp, _vp, _int, _int]
        lib.oracle_squared_relu_probs_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                                      _int, ctypes.c_float, _vp, _vp, _int, _int]
        lib.oracle_unpermute_expert_order.argtypes = [_vp, _i64, _vp, _vp, _vp, _int, _i64, _i64, _i64,
                                                      _int]
        for f in ("oracle_residual_add", "oracle_router_weight_fwd", "oracle_router_weight_bwd",
                  "oracle_squared_relu_probs_fwd", "oracle_squared_relu_probs_bwd",
                  "oracle_unpermute_expert_order"):
            getattr(lib, f).restype = ctypes.c_int
        self.lib = lib

    @staticmethod
    def _rc(rc, what):
        if rc != 0:
            raise ValueError(f"{what} rejected its arguments")

    # conversions (own fp16 rounding; pinned against numpy/torch)
    def f16_from_f32(self, a):
        a = _c(a, np.float32)
        out = np.empty(a.shape, np.uint16)
        self.lib.oracle_f16_from_f32(_p(a), _p(out), a.size)
        return out

    def f32_from_f16(self, a):
        a = _c(a, np.uint16)
        out = np.empty(a.shape, np.float32)
        self.lib.oracle_f32_from_f16(_p(a), _p(out), a.size)
        return out

    def residual_add(self, expert, shared, residual, dtype: str, threads: Optional[int] = None):
        e, s, r = (_c(v, NP[dtype]) for v in (expert, shared, residual))
        if not (e.shape == s.shape == r.shape):
            raise ValueError("shape mismatch")
        out = np.empty_like(e)
        self._rc(self.lib.oracle_residual_add(_p(e), _p(s), _p(r), _p(out), e.size, DTYPES[dtype],
                                              threads or default_threads()), "oracle_residual_add")
        return out

    def router_weight_fwd(self, x, x_dtype: str, probs, out_dtype: str, threads: Optional[int] = None):
        x = _c(x, NP[x_dtype])
        tokens, hidden = x.shape
        probs = _c(np.asarray(probs).reshape(-1), np.float32)
        out = np.empty((tokens, hidden), NP[out_dtype])
        self._rc(self.lib.oracle_router_weight_fwd(_p(x), DTYPES[x_dtype], _p(probs), _p(out),
                                                   DTYPES[out_dtype], tokens, hidden,
                                                   threads or default_threads()),
                 "oracle_router_weight_fwd")
        return out

    def router_weight_bwd(self, grad_out, out_dtype: str, x, x_dtype: str, probs,
                          want_grad_x=True, want_grad_probs=True, threads: Optional[int] = None):
        g = _c(grad_out, NP[out_dtype])
        tokens, hidden = g.shape
        probs = _c(np.asarray(probs).reshape(-1), np.float32)
        xx = None if x is None else _c(x, NP[x_dtype])
        gx = np.empty((tokens, hidden), NP[x_dtype]) if want_grad_x else None
        gp = gp64 = sc = None
        if want_grad_probs:
            gp = np.empty(tokens, np.float32)
            gp64 = np.empty(tokens, np.float64)
            sc = np.empty(tokens, np.float64)
        self._rc(self.lib.oracle_router_weight_bwd(_p(g), DTYPES[out_dtype], _p(xx), DTYPES[x_dtype],
                                                   _p(probs), _p(gx), _p(gp), _p(gp64), _p(sc),
                                                   tokens, hidden, threads or default_threads()),
                 "oracle_router_weight_bwd")
        return {"grad_x": gx, "grad_probs": gp, "grad_probs_f64": gp64, "row_scale": sc}

    def squared_relu_probs(self, x, probs, *, clamp_scale=None, n_used=None, permutation_map=None,
                           zero_padding=False, out=None, threads: Optional[int] = None):
        x = _c(x, np.uint16)
        rows, hidden = x.shape
        probs = _c(np.asarray(probs).reshape(-1), np.float32)
        y = np.full((rows, hidden), 0xFFFF, np.uint16) if out is None else _c(out, np.uint16)
        nu = None if n_used is None else np.array([n_used], np.int32)
        pm = None if permutation_map is None else _c(permutation_map, np.int32)
        clamp = clamp_scale is not None
        self._rc(self.lib.oracle_squared_relu_probs_fwd(_p(x), _p(probs), _p(y), rows, hidden,
                                                        int(clamp), float(clamp_scale or 0.0), _p(nu),
                                                        _p(pm), int(bool(zero_padding)),
                                                        threads or default_threads()),
                 "oracle_squared_relu_probs_fwd")
        return y

    def squared_relu_probs_bwd(self, x, probs, grad_y, *, clamp_scale=None, n_used=None,
                               permutation_map=None, zero_padding=False, grad_x_out=None,
                               grad_probs_out=None, want_grad_x=True, threads: Optional[int] = None):
        """grad_x (bf16 bits), grad_probs (fp32, slot-indexed), grad_probs_f64 and the row
        scale S = sum |g * y_pre| (both slot-indexed; NaN where a slot is not live)."""
        x = _c(x, np.uint16)
        g = _c(grad_y, np.uint16)
        rows, hidden = x.shape
        if g.shape != x.shape:
            raise ValueError("shape mismatch")
        probs = _c(np.asarray(probs).reshape(-1), np.float32)
        gx = None
        if want_grad_x:
            gx = np.full((rows, hidden), 0xFFFF, np.uint16) if grad_x_out is None \
                else _c(grad_x_out, np.uint16)
        gp = np.full(rows, -12345.5, np.float32) if grad_probs_out is None \
            else _c(grad_probs_out, np.float32)
        gp64 = np.full(rows, np.nan)
        sc = np.full(rows, np.nan)
        nu = None if n_used is None else np.array([n_used], np.int32)
        pm = None if permutation_map is None else _c(permutation_map, np.int32)
        clamp = clamp_scale is not None
        self._rc(self.lib.oracle_squared_relu_probs_bwd(_p(x), _p(probs), _p(g), _p(gx), _p(gp),
                                                        _p(gp64), _p(sc), rows, hidden, int(clamp),
                                                        float(clamp_scale or 0.0), _p(nu), _p(pm),
                                                        int(bool(zero_padding)), threads or default_threads()),
                 "oracle_squared_relu_probs_bwd")
        return {"grad_x": gx, "grad_probs": gp, "grad_probs_f64": gp64, "row_scale": sc}

    def unpermute(self, expert_output, inverse_map, out_dtype: str, *, valid_tokens=None, out=None,
                  threads: Optional[int] = None):
        eo = _c(expert_output, np.uint16)
        expert_rows, hidden = eo.shape
        im = _c(inverse_map, np.int32)
        tokens, n_exp = im.shape
        o = np.full((tokens, hidden), 0xFFFF if out_dtype != "f32" else np.nan, NP[out_dtype]) \
            if out is None else _c(out, NP[out_dtype])
        vt = None if valid_tokens is None else np.array([valid_tokens], np.int32)
        self._rc(self.lib.oracle_unpermute_expert_order(_p(eo), expert_rows, _p(im), _p(vt), _p(o),
                                                        DTYPES[out_dtype], tokens, hidden, n_exp,
                                                        threads or default_threads()),
                 "oracle_unpermute_expert_order")
        return o


_default: Optional[MoeOracle] = None


def get() -> MoeOracle:
    global _default
    if _default is None:
        _default = MoeOracle()
    return _default
