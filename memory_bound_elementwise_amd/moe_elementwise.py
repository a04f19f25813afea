"""Python binding of ``libmoe_elementwise.so`` (C ABI in ``include/moe_elementwise.h``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity and their device pointers and the current HIP stream are handed to the
C functions of the same names. No CPU or PyTorch fallback.

16-bit tensors may be given in their own dtype (bf16 / fp16) or as int16 / uint16
bit patterns together with an explicit ``dtype`` where the call takes one.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

from . import build as _build

MOE_BF16, MOE_FP16, MOE_FP32 = 0, 1, 2
_NAMES = {"bf16": MOE_BF16, "f16": MOE_FP16, "f32": MOE_FP32}
_TORCH = {torch.bfloat16: MOE_BF16, torch.float16: MOE_FP16, torch.float32: MOE_FP32}

_lock = threading.Lock()
_lib = None
_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGS = {
    "moe_residual_add": [_vp, _vp, _vp, _vp, _i64, _int, _vp, _int],
    "moe_router_weight_fwd": [_vp, _int, _vp, _vp, _int, _i64, _i64, _vp, _int],
    "moe_router_weight_bwd": [_vp, _int, _vp, _int, _vp, _vp, _vp, _i64, _i64, _vp, _int],
    "moe_squared_relu_probs_fwd": [_vp, _vp, _vp, _i64, _i64, _int, ctypes.c_float, _vp, _vp, _int,
                                   _vp, _int],
    "moe_squared_relu_probs_bwd": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, ctypes.c_float, _vp, _vp,
                                   _int, _vp, _int],
    "moe_unpermute_expert_order": [_vp, _i64, _vp, _vp, _vp, _int, _i64, _i64, _int, _vp, _int],
    "moe_elementwise_status_string": [_int],
    "moe_elementwise_last_hip_error": [],
    "moe_elementwise_abi_version": [],
}


class MoeElementwiseError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status, self.hip_error = status, hip_error
        msg = load_library().moe_elementwise_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status}" +
                         (f", hipError {hip_error})" if status == 3 else ")"))


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or _build.lib_path("moe_elementwise")
        if not os.path.exists(p):
            _build.build_lib("moe_elementwise")
        lib = ctypes.CDLL(p)
        for name, args in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "moe_elementwise_status_string" else ctypes.c_int
        if lib.moe_elementwise_abi_version() != 1:
            raise RuntimeError("libmoe_elementwise.so ABI version mismatch")
        if path is None:
            _lib = lib
        return lib


def _check(fn, st):
    if st != 0:
        raise MoeElementwiseError(fn, st, load_library().moe_elementwise_last_hip_error())


def _dt(t: torch.Tensor, dtype: Optional[str]) -> int:
    if dtype is not None:
        code = _NAMES[dtype]
        want = 4 if code == MOE_FP32 else 2
        if t.element_size() != want:
            raise TypeError(f"{dtype} tensor expected, got {t.dtype}")
        return code
    if t.dtype not in _TORCH:
        raise TypeError(f"cannot infer the element type of a {t.dtype} tensor; pass dtype=")
    return _TORCH[t.dtype]


def _bf16_bits(name, *ts):
    """bf16 tensors, or int16 / uint16 views of bf16 bit patterns (never fp16: its bits
    would be read as bf16)."""
    for t in ts:
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError(f"{name} must be bf16 (or its int16/uint16 bits), got {t.dtype}")


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must live on one device")
    return dev


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, dev):
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def moe_residual_add(expert_output, shared_expert_output, residual, output, *, dtype=None,
                     stream=None, num_workgroups=0):
    """output = residual + round_to_dtype(expert_output + shared_expert_output)."""
    d = _dt(expert_output, dtype)
    for t in (shared_expert_output, residual, output):
        if t.shape != expert_output.shape or _dt(t, dtype) != d:
            raise ValueError("all four tensors need one shape and one dtype")
    dev = _dev(expert_output, shared_expert_output, residual, output)
    st = load_library().moe_residual_add(_ptr(expert_output), _ptr(shared_expert_output), _ptr(residual),
                                         _ptr(output), expert_output.numel(), d, _stream(stream, dev),
                                         int(num_workgroups))
    _check("moe_residual_add", st)
    return output


def moe_router_weight_fwd(x, probs, out, *, x_dtype=None, out_dtype=None, stream=None,
                          num_workgroups=0):
    """out = (x.float() * probs.float()).to(out dtype); x and out are [tokens, hidden]."""
    if x.dim() != 2 or out.shape != x.shape:
        raise ValueError("x and out must be [tokens, hidden]")
    if probs.dtype != torch.float32 or probs.numel() != x.shape[0]:
        raise ValueError("probs must be fp32 with one value per token")
    dev = _dev(x, probs, out)
    st = load_library().moe_router_weight_fwd(_ptr(x), _dt(x, x_dtype), _ptr(probs), _ptr(out),
                                              _dt(out, out_dtype), x.shape[0], x.shape[1],
                                              _stream(stream, dev), int(num_workgroups))
    _check("moe_router_weight_fwd", st)
    return out


def moe_router_weight_bwd(grad_out, x, probs, grad_x, grad_probs, *, out_dtype=None, x_dtype=None,
                          stream=None, num_workgroups=0):
    """grad_x = (grad_out.float() * probs).to(x dtype); grad_probs = sum(grad_out * x, -1) in fp32.
    ``x`` may be None when ``grad_probs`` is None; either output may be None."""
    if grad_out.dim() != 2:
        raise ValueError("grad_out must be [tokens, hidden]")
    tokens, hidden = grad_out.shape
    xd = _dt(x, x_dtype) if x is not None else (_dt(grad_x, x_dtype) if grad_x is not None
                                                 else _NAMES.get(x_dtype or "bf16"))
    for t in (x, grad_x):
        if t is not None and t.shape != grad_out.shape:
            raise ValueError("x and grad_x must match grad_out's shape")
    if probs.dtype != torch.float32 or probs.numel() != tokens:
        raise ValueError("probs must be fp32 with one value per token")
    if grad_probs is not None and (grad_probs.dtype != torch.float32 or grad_probs.numel() != tokens):
        raise ValueError("grad_probs must be fp32 with one value per token")
    dev = _dev(grad_out, x, probs, grad_x, grad_probs)
    st = load_library().moe_router_weight_bwd(_ptr(grad_out), _dt(grad_out, out_dtype), _ptr(x), xd,
                                              _ptr(probs), _ptr(grad_x), _ptr(grad_probs), tokens,
                                              hidden, _stream(stream, dev), int(num_workgroups))
    _check("moe_router_weight_bwd", st)
    return grad_x, grad_probs


def moe_squared_relu_probs_fwd(x, probs, y, *, clamp_scale=None, n_used=None, permutation_map=None,
                               zero_padding=False, stream=None, num_workgroups=0):
    """Squared ReLU x probs (bf16 in and out); ``clamp_scale`` enables the tanh soft clamp."""
    _bf16_bits("x and y", x, y)
    if x.dim() != 2 or y.shape != x.shape:
        raise ValueError("x and y must be bf16 [rows, hidden]")
    rows, hidden = x.shape
    if probs.dtype != torch.float32 or probs.numel() != rows:
        raise ValueError("probs must be fp32 with one value per row")
    if n_used is not None and (n_used.dtype != torch.int32 or n_used.numel() != 1):
        raise ValueError("n_used must be a device int32 scalar")
    if permutation_map is not None and (permutation_map.dtype != torch.int32 or
                                        permutation_map.numel() != rows):
        raise ValueError("permutation_map must be int32 [rows]")
    dev = _dev(x, probs, y, n_used, permutation_map)
    clamp = clamp_scale is not None
    st = load_library().moe_squared_relu_probs_fwd(_ptr(x), _ptr(probs), _ptr(y), rows, hidden,
                                                   int(clamp), float(clamp_scale if clamp else 0.0),
                                                   _ptr(n_used), _ptr(permutation_map),
                                                   int(bool(zero_padding)), _stream(stream, dev),
                                                   int(num_workgroups))
    _check("moe_squared_relu_probs_fwd", st)
    return y


def moe_squared_relu_probs_bwd(x, probs, grad_y, grad_x, grad_probs=None, *, clamp_scale=None,
                               n_used=None, permutation_map=None, zero_padding=False, stream=None,
                               num_workgroups=0):
    """Backward of ``moe_squared_relu_probs_fwd``: grad_x (bf16) and, when given, grad_probs
    (fp32 [rows], indexed by slot; slots of rows that are not live are left as they are)."""
    _bf16_bits("x, grad_y and grad_x", x, grad_y, grad_x)
    if x.dim() != 2 or grad_y.shape != x.shape or grad_x.shape != x.shape:
        raise ValueError("x, grad_y and grad_x must be bf16 [rows, hidden]")
    rows, hidden = x.shape
    if probs.dtype != torch.float32 or probs.numel() != rows:
        raise ValueError("probs must be fp32 with one value per row")
    if grad_probs is not None and (grad_probs.dtype != torch.float32 or grad_probs.numel() != rows):
        raise ValueError("grad_probs must be fp32 with one value per row")
    if n_used is not None and (n_used.dtype != torch.int32 or n_used.numel() != 1):
        raise ValueError("n_used must be a device int32 scalar")
    if permutation_map is not None and (permutation_map.dtype != torch.int32 or
                                        permutation_map.numel() != rows):
        raise ValueError("permutation_map must be int32 [rows]")
    dev = _dev(x, probs, grad_y, grad_x, grad_probs, n_used, permutation_map)
    clamp = clamp_scale is not None
    st = load_library().moe_squared_relu_probs_bwd(_ptr(x), _ptr(probs), _ptr(grad_y), _ptr(grad_x),
                                                   _ptr(grad_probs), rows, hidden, int(clamp),
                                                   float(clamp_scale if clamp else 0.0), _ptr(n_used),
                                                   _ptr(permutation_map), int(bool(zero_padding)),
                                                   _stream(stream, dev), int(num_workgroups))
    _check("moe_squared_relu_probs_bwd", st)
    return grad_x, grad_probs


def moe_unpermute_expert_order(expert_output, inverse_map, out, *, valid_tokens=None,
                               out_dtype=None, stream=None, num_workgroups=0):
    """out[t] = sum over local experts e in increasing order of expert_output[inverse_map[t, e]]."""
    _bf16_bits("expert_output", expert_output)
    if expert_output.dim() != 2:
        raise ValueError("expert_output must be bf16 [rows, hidden]")
    if inverse_map.dim() != 2 or inverse_map.dtype != torch.int32:
        raise ValueError("inverse_map must be int32 [tokens, num_local_experts]")
    tokens, n_exp = inverse_map.shape
    if out.shape != (tokens, expert_output.shape[1]):
        raise ValueError("out must be [tokens, hidden]")
    if valid_tokens is not None and (valid_tokens.dtype != torch.int32 or valid_tokens.numel() != 1):
        raise ValueError("valid_tokens must be a device int32 scalar")
    dev = _dev(expert_output, inverse_map, out, valid_tokens)
    st = load_library().moe_unpermute_expert_order(_ptr(expert_output), expert_output.shape[0],
                                                   _ptr(inverse_map), _ptr(valid_tokens), _ptr(out),
                                                   _dt(out, out_dtype), tokens, expert_output.shape[1],
                                                   n_exp, _stream(stream, dev), int(num_workgroups))
    _check("moe_unpermute_expert_order", st)
    return out


class FusedMoEResidualAdd(torch.autograd.Function):
    """residual + (expert_output + shared_expert_output), one fused launch. Each input enters
    the sum with weight one, so the backward hands the incoming gradient to all of them."""

    @staticmethod
    def forward(ctx, expert_output, shared_expert_output, residual):
        return moe_residual_add(expert_output, shared_expert_output, residual,
                                torch.empty_like(residual))

    @staticmethod
    def backward(ctx, grad_output):
        return grad_output, grad_output, grad_output


class RouterWeightMul(torch.autograd.Function):
    """(x.float() * probs.float()).to(out_dtype) saving only the low-precision inputs; the
    backward recomputes nothing and reads x only when probs needs a gradient."""

    @staticmethod
    def forward(ctx, x, probs, out_dtype):
        save_x = probs.requires_grad
        ctx.save_for_backward(x if save_x else None, probs)
        ctx.x_dtype = x.dtype
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
        return moe_router_weight_fwd(x, probs, out)

    @staticmethod
    def backward(ctx, grad_out):
        x, probs = ctx.saved_tensors
        grad_out = grad_out.contiguous()
        gx = torch.empty(grad_out.shape, dtype=ctx.x_dtype, device=grad_out.device) \
            if ctx.needs_input_grad[0] else None
        gp = torch.empty(probs.shape, dtype=torch.float32, device=grad_out.device) \
            if ctx.needs_input_grad[1] else None
        moe_router_weight_bwd(grad_out, x, probs, gx, gp,
                              x_dtype={torch.bfloat16: "bf16", torch.float16: "f16",
                                       torch.float32: "f32"}[ctx.x_dtype])
        return gx, gp, None


class SquaredReluProbs(torch.autograd.Function):
    """relu(x)^2 * probs, or relu(s * tanh(x / s))^2 * probs with ``clamp_scale`` s, in the
    HIP kernels. Saves only ``x`` and ``probs``; the backward recomputes the activation.
    ``x`` bf16 [rows, hidden] contiguous, ``probs`` fp32 [rows] or [rows, 1]; every row live."""

    @staticmethod
    def forward(ctx, x, probs, clamp_scale=None):
        ctx.save_for_backward(x, probs)
        ctx.clamp_scale = clamp_scale
        return moe_squared_relu_probs_fwd(x, probs.reshape(-1), torch.empty_like(x),
                                          clamp_scale=clamp_scale)

    @staticmethod
    def backward(ctx, grad_y):
        x, probs = ctx.saved_tensors
        gx = torch.empty_like(x)
        gp = torch.empty(probs.numel(), dtype=torch.float32, device=x.device) \
            if ctx.needs_input_grad[1] else None
        moe_squared_relu_probs_bwd(x, probs.reshape(-1), grad_y.contiguous(), gx, gp,
                                   clamp_scale=ctx.clamp_scale)
        return gx, (None if gp is None else gp.view(probs.shape)), None
