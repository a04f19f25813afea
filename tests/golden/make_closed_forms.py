"""Write ``closed_forms.json``: single-element cases whose results follow from calculus.

The pages print no worked example for the activation, so these fixtures hold
special points where the value of every output is known in closed form:
silu(0) = 0 and silu'(0) = 1/2; silu(z) = z / (1 + e^-z) at a few points;
silu'(z) = sig(z) * (1 + z * (1 - sig(z))); the clamp masks are inclusive
(torch.clamp's gradient convention, NeMo AutoModel "moe/swiglu_triton" page,
module docstring). The values are evaluated here with Python floats (fp64) and
math.exp, then rounded once to bf16 by torch's fp32 -> bf16 cast; neither the
oracle nor the HIP library is involved. Each case records its derivation.

Run: python tests/golden/make_closed_forms.py
"""
from __future__ import annotations

import json
import math
import os

import torch


def bf16_hex(v: float) -> str:
    t = torch.tensor([v], dtype=torch.float64).to(torch.bfloat16)
    return "0x%04X" % (t.view(torch.int16).item() & 0xFFFF)


def bits_hex(v: float) -> str:
    # exact bf16 inputs only
    t = torch.tensor([v], dtype=torch.float32).to(torch.bfloat16)
    assert float(t.to(torch.float32)) == v, v
    return "0x%04X" % (t.view(torch.int16).item() & 0xFFFF)


def sig(z: float) -> float:
    return 1.0 / (1.0 + math.exp(-z))


def case(name, gate, up, p, g, limit, derivation):
    cg = min(gate, limit)
    cu = max(-limit, min(up, limit))
    s = cg * sig(cg)
    ds = sig(cg) * (1.0 + cg * (1.0 - sig(cg)))
    y = s * cu * p
    d_gate = g * p * cu * ds if gate <= limit else 0.0
    d_up = g * p * s if -limit <= up <= limit else 0.0
    return {
        "name": name, "derivation": derivation,
        "gate": gate, "up": up, "p": p, "grad_y": g, "limit": limit,
        "gate_bits": bits_hex(gate), "up_bits": bits_hex(up), "grad_y_bits": bits_hex(g),
        "y": y, "y_bits": bf16_hex(y),
        "d_gate": d_gate, "d_gate_bits": bf16_hex(d_gate),
        "d_up": d_up, "d_up_bits": bf16_hex(d_up),
        "grad_probs": g * s * cu,
    }


CASES = [
    case("gate_zero", 0.0, 3.0, 0.5, 1.0, 7.0,
         "silu(0)=0 so y=0 and d_up=0; silu'(0)=1/2 so d_gate=g*p*up/2=0.75; grad_probs=0"),
    case("gate_at_limit", 7.0, 1.0, 1.0, 1.0, 7.0,
         "gate=L is inside the inclusive mask: d_gate=silu'(7)=1.00546...; y=d_up=silu(7)=6.99362..."),
    case("gate_one_step_above_limit", 7.03125, 1.0, 1.0, 1.0, 7.0,
         "gate=7+1 bf16 ulp clamps to 7 (y=silu(7)) and falls outside the mask: d_gate=0"),
    case("up_at_minus_limit", 1.0, -7.0, 1.0, 1.0, 7.0,
         "up=-L is inside the inclusive mask: d_up=silu(1)=0.73106; y=-7*silu(1); d_gate=-7*silu'(1)"),
    case("up_one_step_below_minus_limit", 1.0, -7.03125, 1.0, 1.0, 7.0,
         "up=-(7+1 ulp) clamps to -7 and falls outside the mask: d_up=0; d_gate as at up=-7"),
    case("unclamped_large", 10.0, 20.0, 0.25, -2.0, math.inf,
         "L=inf: plain silu(10)*20*0.25; d_gate=-0.5*20*silu'(10); d_up=-0.5*silu(10)"),
    case("large_negative_gate", -20.0, 5.0, 1.0, 1.0, 7.0,
         "gate has no lower clamp: silu(-20)=-20/(1+e^20)=-4.1223e-8"),
    case("gate_at_silu_minimum", -1.28125, 2.0, 0.5, 1.0, 7.0,
         "silu' crosses zero near -1.2785; at -1.28125 it is -6.1e-4, so d_gate is tiny and negative"),
]

if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "closed_forms.json")
    with open(out, "w") as fh:
        json.dump({"source": "calculus at special points; see make_closed_forms.py",
                   "cases": CASES}, fh, indent=1)
    print(out)
