"""MI355X-native fused clamped-SwiGLU x routing-probability expert activation.

The activation (forward and backward) runs in hand-written HIP kernels for gfx950
behind the C ABI of ``include/swiglu_probs.h``; this package holds the kernels'
sources (``csrc/``), their in-tree build (``build.py``), the ctypes binding
(``swiglu_probs``), the binding of the MoE elementwise operations next to the
activation (``moe_elementwise``: fused residual add, router-weight multiply,
squared-ReLU x probs forward and backward, unpermute in expert order), the HBM probe binding
(``hbm_probe``) and the seeded input generators (``workloads``). Libraries are
loaded on first use, not at import.
"""
from .swiglu_probs import (SwigluProbs, SwigluProbsError, backward, forward,  # noqa: F401
                           load_library, swiglu_probs_bwd, swiglu_probs_default_workgroups,
                           swiglu_probs_fwd)

from .moe_elementwise import (FusedMoEResidualAdd, MoeElementwiseError,  # noqa: F401
                              RouterWeightMul, SquaredReluProbs, moe_residual_add,
                              moe_router_weight_bwd, moe_router_weight_fwd,
                              moe_squared_relu_probs_bwd, moe_squared_relu_probs_fwd,
                              moe_unpermute_expert_order)

__all__ = ["moe_residual_add", "moe_router_weight_fwd", "moe_router_weight_bwd",
           "moe_squared_relu_probs_fwd", "moe_squared_relu_probs_bwd", "moe_unpermute_expert_order",
           "FusedMoEResidualAdd", "RouterWeightMul", "SquaredReluProbs", "MoeElementwiseError",
           "swiglu_probs_fwd", "swiglu_probs_bwd", "swiglu_probs_default_workgroups",
           "forward", "backward", "SwigluProbs", "SwigluProbsError", "load_library"]
