"""Seeded synthetic inputs for the clamped SwiGLU x probs activation and for the MoE
elementwise operations beside it (``make_moe_inputs``), with their algorithmic byte
counts.

This module draws inputs only; it holds none of the operations' arithmetic and
serves both the HIP path and the CPU oracle (through the tests and the bench).
Every array is drawn on the CPU from ``torch.Generator().manual_seed(seed)`` in
a fixed order, so both sides see the same bytes:

1. ``x``      fp32 draw, scaled, then rounded to bf16 by torch (the input dtype);
2. ``probs``  (for the padded workload: drawn from logits after ``grad_y``);
3. ``grad_y`` fp32 N(0, 1) rounded to bf16;
4. workload-specific draws (edge-value masks, zeroed probabilities, router
   logits, the permutation).

The workloads stand in for the one shape the pages name (one GPU's share of the
routed-expert activation in a 16-node deployment, whose backward moves about 1.1 GB;
NeMo AutoModel "moe/swiglu_triton" page, module docstring) and for the padded inference layout of the Megatron-Core
"core.inference.moe.batch_invariant" page (swiglu_with_probs: permutation_map,
n_used, zero_padding). Arrays are numpy: bf16 values as uint16 bit patterns,
probabilities fp32, the map int32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# bf16 bit patterns used by the edge workload: +7, -7 and 7 + 1 bf16 ulp.
BF16_POS7 = 0x40E0
BF16_NEG7 = 0xC0E0
BF16_POS7_NEXT = 0x40E1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    rows: int
    inter: int
    limit: float
    x_std: float
    probs: str = "uniform"          # "uniform" | "topk_softmax"
    n_used: Optional[int] = None
    permute: bool = False
    zero_padding: bool = False
    edge_fraction: float = 0.0      # fraction of gate/up entries set to an edge value
    zero_prob_fraction: float = 0.0  # fraction of probabilities set exactly to 0
    topk: int = 8
    n_experts: int = 64

    def fwd_bytes(self, rows: Optional[int] = None) -> int:
        """Algorithmic bytes of one forward pass (see ``algorithmic_bytes``)."""
        return algorithmic_bytes(self, "fwd", rows)

    def bwd_bytes(self, rows: Optional[int] = None) -> int:
        return algorithmic_bytes(self, "bwd", rows)


WORKLOADS = {
    "tiny": Workload("tiny", rows=256, inter=256, limit=7.0, x_std=3.0),
    "mid": Workload("mid", rows=16384, inter=2048, limit=7.0, x_std=3.0),
    "headline": Workload("headline", rows=53760, inter=2048, limit=7.0, x_std=3.0),
    "padded": Workload("padded", rows=32768, inter=1536, limit=math.inf, x_std=1.0,
                       probs="topk_softmax", n_used=30000, permute=True, zero_padding=True),
    "edge": Workload("edge", rows=131071, inter=1408, limit=7.0, x_std=3.0,
                     edge_fraction=0.01, zero_prob_fraction=0.05),
}


def live_rows(w: Workload, rows: Optional[int] = None) -> int:
    rows = w.rows if rows is None else rows
    return rows if w.n_used is None else max(0, min(w.n_used, rows))


def algorithmic_bytes(w: Workload, direction: str, rows: Optional[int] = None) -> int:
    """Bytes the method must move for one pass, counting each byte once.

    forward : live*(4*inter + 4 [+4 map]) read + W*2*inter written
    backward: live*(6*inter + 4 [+4 map]) read + W*4*inter + live*4 written
    where W = rows written (all rows with zero_padding, else the live rows) and a
    device n_used adds 4 bytes read.
    """
    rows = w.rows if rows is None else rows
    live = live_rows(w, rows)
    written = rows if w.zero_padding else live
    extra = (4 if w.permute else 0)
    nu = 4 if w.n_used is not None else 0
    if direction == "fwd":
        return live * (4 * w.inter + 4 + extra) + written * 2 * w.inter + nu
    if direction == "bwd":
        return live * (6 * w.inter + 4 + extra) + written * 4 * w.inter + live * 4 + nu
    raise ValueError(direction)


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_inputs(w: Workload | str, seed: int = 0, rows: Optional[int] = None) -> dict:
    """Draw one input set for workload ``w``.

    ``rows`` overrides the row count (the other parameters stay), for reduced
    copies of a workload in fast tests; for the padded workload the live count
    keeps its ratio to the row count.

    Returns a dict with ``x`` (uint16 [rows, 2*inter]), ``probs`` (float32 [rows]),
    ``grad_y`` (uint16 [rows, inter]), ``limit`` (float), ``n_used`` (int or None),
    ``permutation_map`` (int32 [rows] or None), ``zero_padding`` (bool), ``workload``.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    rows = w.rows if rows is None else int(rows)
    inter = w.inter
    g = torch.Generator(device="cpu").manual_seed(seed)

    x32 = torch.randn(rows, 2 * inter, generator=g, dtype=torch.float32)
    if w.x_std != 1.0:
        x32.mul_(w.x_std)
    x = _bf16_bits(x32)
    del x32

    probs = None
    if w.probs == "uniform":
        probs = torch.rand(rows, generator=g, dtype=torch.float32).numpy()
    grad_y = _bf16_bits(torch.randn(rows, inter, generator=g, dtype=torch.float32))

    n_used = None
    perm = None
    if w.edge_fraction > 0.0:
        # Each gate and up entry independently becomes, with probability
        # edge_fraction, one of +7, -7 or 7 + 1 ulp, chosen uniformly.
        hit = torch.rand(rows, 2 * inter, generator=g) < w.edge_fraction
        pick = torch.randint(0, 3, (rows, 2 * inter), generator=g)
        choices = torch.tensor([BF16_POS7, BF16_NEG7 - 65536, BF16_POS7_NEXT], dtype=torch.int32)
        vals = choices[pick].to(torch.int16).numpy().view(np.uint16)
        hitn = hit.numpy()
        x[hitn] = vals[hitn]
    if w.zero_prob_fraction > 0.0:
        zmask = (torch.rand(rows, generator=g) < w.zero_prob_fraction).numpy()
        probs[zmask] = 0.0
    if w.probs == "topk_softmax":
        # Router weights: softmax over n_experts logits ~ N(0, 1) per token, keep
        # the top-k weights (no renormalisation), flattened token-major.
        tokens = -(-rows // w.topk)
        logits = torch.randn(tokens, w.n_experts, generator=g, dtype=torch.float32)
        top = torch.softmax(logits, dim=-1).topk(w.topk, dim=-1).values
        probs = top.reshape(-1)[:rows].contiguous().numpy()
    if w.n_used is not None:
        n_used = max(0, min(rows, round(w.n_used * rows / w.rows)))
    if w.permute:
        perm = torch.randperm(rows, generator=g).to(torch.int32).numpy()

    return {
        "x": np.ascontiguousarray(x),
        "probs": np.ascontiguousarray(probs, dtype=np.float32),
        "grad_y": np.ascontiguousarray(grad_y),
        "limit": float(w.limit),
        "n_used": n_used,
        "permutation_map": perm,
        "zero_padding": bool(w.zero_padding),
        "workload": w,
    }


# ---------------------------------------------------------------------------
# Workloads of the MoE elementwise operations next to the activation. Shapes follow
# the headline activation workload: 53760 routed rows = 6720 tokens x top-8, a model
# hidden size of 7168 beside the expert width of 2048, 8 local experts per GPU.
# ---------------------------------------------------------------------------
MOE_TOKENS = 6720
MOE_TOPK = 8
MOE_HIDDEN = 7168
MOE_LOCAL_EXPERTS = 8


def make_moe_inputs(op: str, seed: int = 0, scale: float = 1.0) -> dict:
    """Seeded inputs for one MoE op. ``scale`` < 1 shrinks the token/row count (tests).

    residual_add : expert, shared, residual bf16 [6720, 7168] ~ N(0,1) (residual N(0, 4^2))
    router_weight: x bf16 [53760, 7168] ~ N(0,1), probs U(0,1), grad_out bf16 ~ N(0,1)
    squared_relu : x bf16 [53760, 2048] ~ N(0, 3^2), probs U(0,1), soft clamp scale 4,
                   grad_y bf16 [53760, 2048] ~ N(0, 1) for the backward
    unpermute    : 6720 tokens x 8 local experts, each (token, expert) pair routed with
                   probability 1/2; expert_output bf16 [routed pairs, 7168] ~ N(0,1) in
                   expert-major (grouped-GEMM) order; inverse_map int32 [6720, 8]
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    tokens = max(1, int(MOE_TOKENS * scale))
    rows = tokens * MOE_TOPK

    def bf16(shape, std=1.0):
        t = torch.randn(*shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return _bf16_bits(t)

    if op == "residual_add":
        return {"expert": bf16((tokens, MOE_HIDDEN)), "shared": bf16((tokens, MOE_HIDDEN)),
                "residual": bf16((tokens, MOE_HIDDEN), 4.0)}
    if op == "router_weight":
        x = bf16((rows, MOE_HIDDEN))
        probs = torch.rand(rows, generator=g, dtype=torch.float32).numpy()
        return {"x": x, "probs": probs, "grad_out": bf16((rows, MOE_HIDDEN))}
    if op == "squared_relu":
        x = bf16((rows, 2048), 3.0)
        probs = torch.rand(rows, generator=g, dtype=torch.float32).numpy()
        return {"x": x, "probs": probs, "clamp_scale": 4.0, "grad_y": bf16((rows, 2048))}
    if op == "unpermute":
        valid = (torch.rand(tokens, MOE_LOCAL_EXPERTS, generator=g) < 0.5).numpy()
        im = np.full((tokens, MOE_LOCAL_EXPERTS), -1, np.int32)
        row = 0
        for e in range(MOE_LOCAL_EXPERTS):
            ts = np.flatnonzero(valid[:, e])
            im[ts, e] = np.arange(row, row + ts.size, dtype=np.int32)
            row += ts.size
        return {"expert_output": bf16((max(row, 1), MOE_HIDDEN)), "inverse_map": im}
    raise ValueError(op)


def moe_algorithmic_bytes(op: str, inp: dict, direction: str = "fwd") -> int:
    """Bytes one launch must move (each byte once)."""
    if op == "residual_add":
        return 4 * inp["expert"].size * 2
    if op == "router_weight":
        n, rows = inp["x"].size, inp["x"].shape[0]
        if direction == "fwd":
            return n * 2 + n * 2 + rows * 4                  # read x, write out, read probs
        return n * 2 * 3 + rows * 8                          # read g and x, write grad_x; probs, grad_probs
    if op == "squared_relu":
        n, rows = inp["x"].size, inp["x"].shape[0]
        if direction == "fwd":
            return n * 2 * 2 + rows * 4                      # read x, write y; probs
        return n * 2 * 3 + rows * 8                          # read x and grad_y, write grad_x; probs, grad_probs
    if op == "unpermute":
        im = inp["inverse_map"]
        contrib = int((im >= 0).sum())
        hidden = inp["expert_output"].shape[1]
        return contrib * hidden * 2 + im.shape[0] * hidden * 4 + im.size * 4   # fp32 out
    raise ValueError(op)
