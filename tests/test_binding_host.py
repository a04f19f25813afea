"""The Python bindings check types, shapes and placement before any call into the
libraries, so these run on the host with CPU tensors and never reach HIP."""
import pytest
import torch

from memory_bound_elementwise_amd import (moe_residual_add, moe_router_weight_fwd,
                                          moe_squared_relu_probs_bwd, moe_squared_relu_probs_fwd,
                                          moe_unpermute_expert_order, swiglu_probs_bwd,
                                          swiglu_probs_fwd)

R, H = 4, 16


def _t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_activation_rejects_fp16_and_bad_shapes():
    p = _t((R,), torch.float32)
    with pytest.raises(TypeError):
        swiglu_probs_fwd(_t((R, 2 * H), torch.float16), p, _t((R, H), torch.bfloat16), 7.0)
    with pytest.raises(ValueError):
        swiglu_probs_fwd(_t((R, 2 * H), torch.bfloat16), p, _t((R, 2 * H), torch.bfloat16), 7.0)
    with pytest.raises(ValueError):                 # probs of the wrong length
        swiglu_probs_fwd(_t((R, 2 * H), torch.bfloat16), _t((R + 1,), torch.float32),
                         _t((R, H), torch.bfloat16), 7.0)
    with pytest.raises(ValueError):                 # host tensors: the kernels need the GPU
        swiglu_probs_fwd(_t((R, 2 * H), torch.bfloat16), p, _t((R, H), torch.bfloat16), 7.0)
    with pytest.raises(TypeError):
        swiglu_probs_bwd(_t((R, 2 * H), torch.bfloat16), p, _t((R, H), torch.float16),
                         _t((R, 2 * H), torch.bfloat16), None, 7.0)
    with pytest.raises(ValueError):                 # grad_probs must be fp32
        swiglu_probs_bwd(_t((R, 2 * H), torch.bfloat16), p, _t((R, H), torch.bfloat16),
                         _t((R, 2 * H), torch.bfloat16), _t((R,), torch.float64), 7.0)


def test_squared_relu_rejects_fp16():
    p = _t((R,), torch.float32)
    with pytest.raises(TypeError):
        moe_squared_relu_probs_fwd(_t((R, H), torch.float16), p, _t((R, H), torch.bfloat16))
    with pytest.raises(TypeError):
        moe_squared_relu_probs_fwd(_t((R, H), torch.bfloat16), p, _t((R, H), torch.float16))
    with pytest.raises(TypeError):
        moe_squared_relu_probs_bwd(_t((R, H), torch.bfloat16), p, _t((R, H), torch.float16),
                                   _t((R, H), torch.bfloat16))
    with pytest.raises(ValueError):                 # int16 bits are accepted, host placement is not
        moe_squared_relu_probs_fwd(_t((R, H), torch.int16), p, _t((R, H), torch.int16))


def test_unpermute_and_router_checks():
    with pytest.raises(TypeError):
        moe_unpermute_expert_order(_t((R, H), torch.float16), _t((R, 2), torch.int32),
                                   _t((R, H), torch.float32))
    with pytest.raises(ValueError):                 # map must be int32
        moe_unpermute_expert_order(_t((R, H), torch.bfloat16), _t((R, 2), torch.int64),
                                   _t((R, H), torch.float32))
    with pytest.raises(ValueError):                 # out of the wrong width
        moe_unpermute_expert_order(_t((R, H), torch.bfloat16), _t((R, 2), torch.int32),
                                   _t((R, H + 8), torch.float32))
    with pytest.raises(ValueError):
        moe_router_weight_fwd(_t((R, H), torch.bfloat16), _t((R,), torch.float16),
                              _t((R, H), torch.bfloat16))
    with pytest.raises(ValueError):                 # shapes differ
        moe_residual_add(_t((R, H), torch.bfloat16), _t((R, H + 8), torch.bfloat16),
                         _t((R, H), torch.bfloat16), _t((R, H), torch.bfloat16))
    with pytest.raises(TypeError):                  # int16 bits need an explicit dtype
        moe_residual_add(_t((R, H), torch.int16), _t((R, H), torch.int16),
                         _t((R, H), torch.int16), _t((R, H), torch.int16))
