"""Run the HIP path and the CPU oracle on the same inputs and compare them.

Test infrastructure. The bar:
  * y and grad_x of live rows: within 1 bf16 ulp (+0 == -0, NaN == NaN);
  * rows that are not live: bit-exact (0x0000 with zero_padding, else the sentinel
    the output was filled with before the call);
  * grad_probs of live slots: |gpu - oracle| <= 1e-6 + 1e-5 * S, S = the row's
    sum of |grad_y * silu(cg) * cu| (fp64, from the oracle); when the oracle's fp32
    result is not finite the GPU must give the same class (NaN, +inf or -inf);
  * grad_probs slots no live row maps to: untouched (bit-exact sentinel).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from bf16cmp import grad_probs_violations, ulp_distance
from memory_bound_elementwise_amd import swiglu_probs_bwd, swiglu_probs_fwd

SENTINEL_BITS = 0xFFFF          # a bf16 NaN pattern no kernel produces from finite data
SENTINEL_GP = np.float32(-12345.5)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bits(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def live_mask(inp: dict) -> np.ndarray:
    rows = inp["x"].shape[0]
    bound = rows if inp["n_used"] is None else max(0, min(rows, inp["n_used"]))
    live = np.arange(rows) < bound
    pm = inp["permutation_map"]
    if pm is not None:
        live &= (pm >= 0) & (pm < rows)
    return live


def run_gpu(inp: dict, device="cuda:0", num_workgroups: int = 0, stream=None,
            do_fwd=True, do_bwd=True, grad_probs=True):
    """Returns (y_bits, grad_x_bits, grad_probs) as numpy arrays after one call each."""
    x = to_dev_bits(inp["x"], device)
    probs = torch.from_numpy(inp["probs"]).to(device)
    rows, two_inter = inp["x"].shape
    n_used = None if inp["n_used"] is None else torch.tensor([inp["n_used"]], dtype=torch.int32,
                                                              device=device)
    pm = None if inp["permutation_map"] is None else torch.from_numpy(inp["permutation_map"]).to(device)
    kw = dict(n_used=n_used, permutation_map=pm, zero_padding=inp["zero_padding"],
              num_workgroups=num_workgroups, stream=stream)
    y_np = gx_np = gp_np = None
    if do_fwd:
        y = torch.full((rows, two_inter // 2), -1, dtype=torch.int16, device=device)
        swiglu_probs_fwd(x, probs, y, inp["limit"], **kw)
        torch.cuda.synchronize()
        y_np = y.cpu().numpy().view(np.uint16)
        del y
    if do_bwd:
        gy = to_dev_bits(inp["grad_y"], device)
        gx = torch.full((rows, two_inter), -1, dtype=torch.int16, device=device)
        gp = torch.full((rows,), float(SENTINEL_GP), dtype=torch.float32, device=device) \
            if grad_probs else None
        swiglu_probs_bwd(x, probs, gy, gx, gp, inp["limit"], **kw)
        torch.cuda.synchronize()
        gx_np = gx.cpu().numpy().view(np.uint16)
        gp_np = gp.cpu().numpy() if grad_probs else None
        del gy, gx, gp
    return y_np, gx_np, gp_np


def run_oracle(inp: dict, do_fwd=True, do_bwd=True):
    orc = oracle.get()
    rows, two_inter = inp["x"].shape
    kw = dict(n_used=inp["n_used"], permutation_map=inp["permutation_map"],
              zero_padding=inp["zero_padding"])
    y = out = None
    if do_fwd:
        y = orc.fwd(inp["x"], inp["probs"], inp["limit"],
                    out=np.full((rows, two_inter // 2), SENTINEL_BITS, dtype=np.uint16), **kw)
    if do_bwd:
        out = orc.bwd(inp["x"], inp["probs"], inp["grad_y"], inp["limit"],
                      grad_x_out=np.full((rows, two_inter), SENTINEL_BITS, dtype=np.uint16),
                      grad_probs_out=np.full(rows, SENTINEL_GP, dtype=np.float32), **kw)
    return y, out


def slots_written(inp: dict) -> np.ndarray:
    rows = inp["x"].shape[0]
    live = live_mask(inp)
    pm = inp["permutation_map"]
    written = np.zeros(rows, dtype=bool)
    written[(pm[live] if pm is not None else np.flatnonzero(live))] = True
    return written


def compare_rows(got: np.ndarray, want: np.ndarray, live: np.ndarray, what: str) -> dict:
    d = ulp_distance(got[live], want[live])
    worst = int(d.max()) if d.size else 0
    n_off = int((d > 1).sum())
    pad_ok = np.array_equal(got[~live], want[~live])
    assert n_off == 0, f"{what}: {n_off} live elements beyond 1 bf16 ulp (max {worst})"
    assert pad_ok, f"{what}: rows that are not live differ from the expected padding/sentinel"
    return {"max_ulp": worst, "frac_1ulp": float((d == 1).mean()) if d.size else 0.0}


def compare_grad_probs(got: np.ndarray, ref: dict, inp: dict, what: str) -> dict:
    written = slots_written(inp)
    want32 = ref["grad_probs"]
    assert np.array_equal(got[~written], want32[~written]), f"{what}: grad_probs slot written for a non-live row"
    g, w32 = got[written], want32[written]
    w64, scale = ref["grad_probs_f64"][written], ref["row_scale"][written]
    fin = np.isfinite(w32)
    if (~fin).any():
        same = (np.isnan(g[~fin]) & np.isnan(w32[~fin])) | (g[~fin] == w32[~fin])
        assert same.all(), f"{what}: non-finite grad_probs differ in class"
    bad = grad_probs_violations(g[fin], w64[fin], scale[fin])
    assert bad.size == 0, (f"{what}: {bad.size} grad_probs rows outside 1e-6 + 1e-5*S; first got "
                           f"{g[fin][bad[0]]} want {w64[fin][bad[0]]} S={scale[fin][bad[0]]}")
    lit = np.abs(g[fin].astype(np.float64) - w64[fin]) > 1e-6 + 1e-5 * np.abs(w64[fin])
    err_s = np.abs(g[fin].astype(np.float64) - w64[fin]) / np.maximum(scale[fin], 1e-300)
    return {"max_err_over_S": float(err_s.max()) if err_s.size else 0.0,
            "literal_rel_fail_frac": float(lit.mean()) if lit.size else 0.0}


def check_parity(inp: dict, device="cuda:0", num_workgroups: int = 0, label: str = "") -> dict:
    say(f"[parity] {label}: GPU fwd/bwd rows={inp['x'].shape[0]} inter={inp['x'].shape[1] // 2} "
        f"workgroups={num_workgroups or 'auto'}")
    y, gx, gp = run_gpu(inp, device, num_workgroups)
    say(f"[parity] {label}: oracle")
    ry, rout = run_oracle(inp)
    live = live_mask(inp)
    inter = inp["x"].shape[1] // 2
    stats = {"y": compare_rows(y, ry, live, f"{label} y"),
             "d_gate": compare_rows(gx[:, :inter], rout["grad_x"][:, :inter], live, f"{label} d_gate"),
             "d_up": compare_rows(gx[:, inter:], rout["grad_x"][:, inter:], live, f"{label} d_up"),
             "grad_probs": compare_grad_probs(gp, rout, inp, f"{label} grad_probs")}
    say(f"[parity] {label}: ok {stats}")
    return stats
