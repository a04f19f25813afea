"""MI355X-native fused clamped-SwiGLU x routing-probability expert activation.

The activation (forward and backward) runs in hand-written HIP kernels for gfx950
behind the C ABI of ``include/swiglu_probs.h``; this package holds the kernels'
sources (``csrc/``), their in-tree build (``build.py``), the ctypes binding
(``swiglu_probs``), the HBM probe binding (``hbm_probe``) and the seeded input
generators (``workloads``). The library is loaded on first use, not at import.
"""
from .swiglu_probs import (SwigluProbs, SwigluProbsError, backward, forward,  # noqa: F401
                           load_library, swiglu_probs_bwd, swiglu_probs_default_workgroups,
                           swiglu_probs_fwd)

__all__ = ["swiglu_probs_fwd", "swiglu_probs_bwd", "swiglu_probs_default_workgroups",
           "forward", "backward", "SwigluProbs", "SwigluProbsError", "load_library"]
