"""Pins of the CPU oracle against values fixed independently of it.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when that build of the oracle disagrees with what the pages and the mathematics
fix. ``test_oracle_pins.py`` runs them on the in-tree oracle;
``test_oracle_mutants.py`` runs them on copies of the C source with a planted
mistake and requires that some pin fails for each.

What pins which part of the oracle:

* ``bf16_rne``                 -> pin_rne_matches_torch (torch's fp32->bf16 cast,
                                  bitwise, incl. every halfway case of a few binades)
* fwd, fp32 path, clamp off    -> pin_unclamped_is_plain_swiglu (L = +inf:
                                  torch F.silu(a)*b*p in fp64, one bf16 rounding)
* fwd, fp32 path, p = 1        -> pin_probs_one_is_bare_activation (torch fp32
                                  silu(clamp(a, max=L)) * clamp(b, -L, L))
* fwd + bwd, fp32 path         -> pin_fp32_path_matches_fp64_autograd (torch fp64
                                  autograd through torch.clamp and F.silu, rounded
                                  once to bf16; grad_probs on the row-scale criterion)
* inclusive clamp masks        -> pin_inclusive_masks (torch fp64 autograd at
                                  exactly +-L and one bf16 step beyond)
* fp64 path                    -> pin_fp64_path_matches_autograd,
                                  pin_fp64_central_differences
* grad_probs                   -> pin_grad_probs_brute_force (Python math.exp loop)
* closed forms                 -> pin_closed_forms (tests/golden/closed_forms.json)
* structure                    -> pin_structure (row-subset invariance, exact
                                  doubling in grad_y, grad_probs independent of p,
                                  p = 0 gives zeros, thread-count invariance)
* row bookkeeping              -> pin_rows_n_used, pin_rows_permutation,
                                  pin_rows_dummy_entries
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from bf16cmp import (assert_within_ulp, bf16_bits_to_f32, grad_probs_violations,
                     ulp_distance)
from memory_bound_elementwise_amd.workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _torch_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _split(x_bits: np.ndarray):
    inter = x_bits.shape[1] // 2
    x = bf16_bits_to_f32(x_bits)
    return x[:, :inter], x[:, inter:]


def torch_autograd_f64(gate, up, probs, grad_y, limit):
    """y, d_gate, d_up, grad_probs from torch float64 autograd of
    silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs."""
    a = torch.tensor(np.asarray(gate, dtype=np.float64), requires_grad=True)
    b = torch.tensor(np.asarray(up, dtype=np.float64), requires_grad=True)
    p = torch.tensor(np.asarray(probs, dtype=np.float64).reshape(-1, 1), requires_grad=True)
    g = torch.tensor(np.asarray(grad_y, dtype=np.float64))
    y = F.silu(torch.clamp(a, max=limit)) * torch.clamp(b, min=-limit, max=limit) * p
    y.backward(g)
    return (y.detach().numpy(), a.grad.numpy(), b.grad.numpy(), p.grad.numpy().reshape(-1))


def _small(seed=0, rows=64, inter=96, limit=7.0, std=3.0):
    g = torch.Generator().manual_seed(seed)
    x = _torch_bf16_bits(torch.randn(rows, 2 * inter, generator=g) * std)
    probs = torch.rand(rows, generator=g).numpy().astype(np.float32)
    gy = _torch_bf16_bits(torch.randn(rows, inter, generator=g))
    return x, probs, gy, limit


# ---------------------------------------------------------------------------
def pin_rne_matches_torch(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # every halfway and near-halfway pattern in a few binades, both signs
    halfway = []
    for exp in (0x3F8, 0x3F0, 0x400, 0x7F0, 0x008, 0x000):
        for mant_hi in range(0, 128, 3):
            base = (exp << 20) | (mant_hi << 16)
            for low in (0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF):
                halfway.append(base | low)
                halfway.append(0x80000000 | base | low)
    special = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001,
               0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x00008000, 0x00018000]
    allbits = np.concatenate([bits, np.array(halfway + special, dtype=np.uint32)])
    f = allbits.view(np.float32)
    got = orc.bf16_rne(f)
    want = _torch_bf16_bits(torch.from_numpy(f.copy()))
    nan = np.isnan(f)
    assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0)), "NaN must stay NaN"
    mism = np.flatnonzero(got[~nan] != want[~nan])
    assert mism.size == 0, (
        f"bf16 rounding differs from torch at {mism.size} inputs; first 0x{int(allbits[~nan][mism[0]]):08x}")


def pin_unclamped_is_plain_swiglu(orc):
    x, probs, gy, _ = _small(seed=2, std=4.0)
    gate, up = _split(x)
    y = orc.fwd(x, probs, math.inf)
    a = torch.tensor(gate, dtype=torch.float64)
    b = torch.tensor(up, dtype=torch.float64)
    p = torch.tensor(probs, dtype=torch.float64).reshape(-1, 1)
    want = _torch_bf16_bits(F.silu(a) * b * p)
    assert_within_ulp(y, want, 1, "fwd with limit=inf vs F.silu(gate)*up*p")
    out = orc.bwd(x, probs, gy, math.inf)
    _, dg, du, dp = torch_autograd_f64(gate, up, probs, bf16_bits_to_f32(gy), math.inf)
    inter = gate.shape[1]
    assert_within_ulp(out["grad_x"][:, :inter], _torch_bf16_bits(torch.from_numpy(dg)), 1, "d_gate, L=inf")
    assert_within_ulp(out["grad_x"][:, inter:], _torch_bf16_bits(torch.from_numpy(du)), 1, "d_up, L=inf")
    bad = grad_probs_violations(out["grad_probs"], dp, out["row_scale"])
    assert bad.size == 0, f"grad_probs, L=inf: {bad.size} rows off"


def pin_probs_one_is_bare_activation(orc):
    x, _, _, limit = _small(seed=3)
    ones = np.ones(x.shape[0], dtype=np.float32)
    gate, up = _split(x)
    y = orc.fwd(x, ones, limit)
    a = torch.from_numpy(gate.copy())
    b = torch.from_numpy(up.copy())
    want = _torch_bf16_bits(F.silu(torch.clamp(a, max=limit)) * torch.clamp(b, -limit, limit))
    assert_within_ulp(y, want, 1, "fwd with p=1 vs torch fp32 silu(clamp)*clamp")


def pin_fp32_path_matches_fp64_autograd(orc):
    for seed, limit, std in ((4, 7.0, 3.0), (5, 2.5, 3.0), (6, 0.75, 1.0)):
        x, probs, gy, _ = _small(seed=seed, limit=limit, std=std)
        gate, up = _split(x)
        yv, dg, du, dp = torch_autograd_f64(gate, up, probs, bf16_bits_to_f32(gy), limit)
        y = orc.fwd(x, probs, limit)
        assert_within_ulp(y, _torch_bf16_bits(torch.from_numpy(yv)), 1, f"fwd L={limit}")
        out = orc.bwd(x, probs, gy, limit)
        inter = gate.shape[1]
        assert_within_ulp(out["grad_x"][:, :inter], _torch_bf16_bits(torch.from_numpy(dg)), 1,
                          f"d_gate L={limit}")
        assert_within_ulp(out["grad_x"][:, inter:], _torch_bf16_bits(torch.from_numpy(du)), 1,
                          f"d_up L={limit}")
        bad = grad_probs_violations(out["grad_probs"], dp, out["row_scale"])
        assert bad.size == 0, f"grad_probs L={limit}: {bad.size} rows off"
        # the fp64 accumulator of fp32 terms is far tighter than the fp32 result
        rel = np.abs(out["grad_probs_f64"] - dp) / out["row_scale"]
        assert np.all(rel < 1e-6), f"fp64 row sums drift from autograd (max {rel.max():.3g} of S)"


def pin_inclusive_masks(orc):
    """d clamp(max=L)/d gate is 1 at gate = L and 0 one step above; d clamp(-L, L)/d up
    is 1 at +-L and 0 one step outside. Checked against torch fp64 autograd."""
    L = 7.0
    vals = np.array([7.0, 7.03125, -7.0, -7.03125, 6.96875, 0.0, -20.0, 100.0], dtype=np.float32)
    n = vals.size
    gate = np.repeat(vals, n).reshape(n, n)      # row i: gate = vals[i]
    up = np.tile(vals, n).reshape(n, n)          # column j: up = vals[j]
    x = np.concatenate([_torch_bf16_bits(torch.from_numpy(gate)),
                        _torch_bf16_bits(torch.from_numpy(up))], axis=1)
    probs = np.full(n, 0.75, dtype=np.float32)
    gy_f = np.full((n, n), 1.5, dtype=np.float32)
    gy = _torch_bf16_bits(torch.from_numpy(gy_f))
    _, dg, du, dp = torch_autograd_f64(gate, up, probs, gy_f, L)
    # the torch reference itself: inclusive at the edges
    assert dg[0, 0] != 0 and np.all(dg[1, :] == 0), "torch reference lost its inclusive gate mask"
    out = orc.bwd(x, probs, gy, L)
    got_dg = bf16_bits_to_f32(out["grad_x"][:, :n]).astype(np.float64)
    got_du = bf16_bits_to_f32(out["grad_x"][:, n:]).astype(np.float64)
    assert np.array_equal(got_dg == 0, dg == 0), "d_gate zero pattern differs from torch.clamp's"
    assert np.array_equal(got_du == 0, du == 0), "d_up zero pattern differs from torch.clamp's"
    assert_within_ulp(out["grad_x"][:, :n], _torch_bf16_bits(torch.from_numpy(dg)), 1, "d_gate at edges")
    assert_within_ulp(out["grad_x"][:, n:], _torch_bf16_bits(torch.from_numpy(du)), 1, "d_up at edges")
    # the same through the fp64 path
    gx64, _ = orc.bwd_f64(np.concatenate([gate, up], axis=1).astype(np.float64), probs,
                          gy_f.astype(np.float64), L)
    assert np.allclose(gx64[:, :n], dg, rtol=1e-12, atol=0), "fp64 d_gate at edges"
    assert np.allclose(gx64[:, n:], du, rtol=1e-12, atol=0), "fp64 d_up at edges"


def pin_fp64_path_matches_autograd(orc):
    rng = np.random.default_rng(7)
    rows, inter, L = 8, 24, 2.0
    x = rng.normal(0, 2.5, size=(rows, 2 * inter))
    probs = rng.uniform(0, 1, size=rows)
    gy = rng.normal(0, 1, size=(rows, inter))
    yv, dg, du, dp = torch_autograd_f64(x[:, :inter], x[:, inter:], probs, gy, L)
    y = orc.fwd_f64(x, probs, L)
    gx, gp = orc.bwd_f64(x, probs, gy, L)
    np.testing.assert_allclose(y, yv, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(gx[:, :inter], dg, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(gx[:, inter:], du, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(gp, dp, rtol=1e-12, atol=1e-14)


def pin_fp64_central_differences(orc):
    """Central differences in fp64 of the loss sum(grad_y * y) agree with the fp64
    backward to 1e-6 relative. Inputs stay at least 1e-3 away from +-L, where the
    clamp has a kink and a central difference averages two one-sided slopes."""
    rng = np.random.default_rng(8)
    rows, inter, L, h = 4, 8, 7.0, 1e-6
    x = rng.normal(0, 3.0, size=(rows, 2 * inter))
    near = np.abs(np.abs(x) - L) < 1e-3
    x[near] += 0.01
    probs = rng.uniform(0.1, 1, size=rows)
    gy = rng.normal(0, 1, size=(rows, inter))
    gx, gp = orc.bwd_f64(x, probs, gy, L)

    def loss(xx, pp):
        return float(np.sum(gy * orc.fwd_f64(xx, pp, L)))

    for r in range(rows):
        for c in range(2 * inter):
            xp, xm = x.copy(), x.copy()
            xp[r, c] += h
            xm[r, c] -= h
            fd = (loss(xp, probs) - loss(xm, probs)) / (2 * h)
            assert abs(fd - gx[r, c]) <= 1e-6 * max(1.0, abs(gx[r, c])), \
                f"FD d x[{r},{c}]: fd={fd} analytic={gx[r, c]}"
        pp, pm = probs.copy(), probs.copy()
        pp[r] += h
        pm[r] -= h
        fd = (loss(x, pp) - loss(x, pm)) / (2 * h)
        assert abs(fd - gp[r]) <= 1e-6 * max(1.0, abs(gp[r])), f"FD d p[{r}]: fd={fd} analytic={gp[r]}"


def pin_grad_probs_brute_force(orc):
    """grad_probs = sum_j grad_y * silu(clamp(gate, max=L)) * clamp(up, -L, L), recomputed
    with Python floats and math.exp on the tiny workload."""
    inp = make_inputs("tiny", seed=0)
    x, probs, gy, L = inp["x"], inp["probs"], inp["grad_y"], inp["limit"]
    gate, up = _split(x)
    g = bf16_bits_to_f32(gy)
    want = np.empty(x.shape[0])
    for r in range(x.shape[0]):
        acc = 0.0
        ga, ub, gr = gate[r].tolist(), up[r].tolist(), g[r].tolist()
        for j in range(len(ga)):
            cg = min(ga[j], L)
            cu = max(-L, min(ub[j], L))
            acc += gr[j] * (cg / (1.0 + math.exp(-cg))) * cu
        want[r] = acc
    out = orc.bwd(x, probs, gy, L)
    bad = grad_probs_violations(out["grad_probs"], want, out["row_scale"])
    assert bad.size == 0, f"grad_probs vs brute force: {bad.size} rows off (first {bad[:3]})"


def pin_closed_forms(orc):
    with open(os.path.join(GOLDEN, "closed_forms.json")) as fh:
        cases = json.load(fh)["cases"]
    for case in cases:
        x = np.array([[int(case["gate_bits"], 16), int(case["up_bits"], 16)]], dtype=np.uint16)
        probs = np.array([case["p"]], dtype=np.float32)
        gy = np.array([[int(case["grad_y_bits"], 16)]], dtype=np.uint16)
        L = float(case["limit"])
        y = orc.fwd(x, probs, L)
        out = orc.bwd(x, probs, gy, L)
        name = case["name"]
        for key, got in (("y_bits", y[0, 0]), ("d_gate_bits", out["grad_x"][0, 0]),
                         ("d_up_bits", out["grad_x"][0, 1])):
            want = int(case[key], 16)
            assert ulp_distance(np.array([got]), np.array([want]))[0] == 0, \
                f"{name}: {key} got 0x{int(got):04x} want 0x{want:04x}"
        gp_want = case["grad_probs"]
        assert abs(float(out["grad_probs"][0]) - gp_want) <= 1e-6 * max(1.0, abs(gp_want)), \
            f"{name}: grad_probs {out['grad_probs'][0]} want {gp_want}"


def pin_structure(orc):
    x, probs, gy, L = _small(seed=9, rows=48, inter=64)
    y = orc.fwd(x, probs, L)
    out = orc.bwd(x, probs, gy, L)
    # rows are independent: a subset in another order gives the same bits
    sub = np.array([5, 0, 47, 13, 13, 2])
    assert np.array_equal(orc.fwd(x[sub], probs[sub], L), y[sub]), "fwd not row-independent"
    o2 = orc.bwd(x[sub], probs[sub], gy[sub], L)
    assert np.array_equal(o2["grad_x"], out["grad_x"][sub]), "bwd not row-independent"
    assert np.array_equal(o2["grad_probs"], out["grad_probs"][sub]), "grad_probs not row-independent"
    # doubling grad_y (exact in bf16 for these magnitudes) doubles every gradient exactly
    gy2 = _torch_bf16_bits(torch.from_numpy(bf16_bits_to_f32(gy) * 2))
    o3 = orc.bwd(x, probs, gy2, L)
    assert np.array_equal(bf16_bits_to_f32(o3["grad_x"]), 2 * bf16_bits_to_f32(out["grad_x"])), \
        "grad_x not linear in grad_y"
    assert np.array_equal(o3["grad_probs"], 2 * out["grad_probs"]), "grad_probs not linear in grad_y"
    # grad_probs does not depend on p
    o4 = orc.bwd(x, probs[::-1].copy(), gy, L)
    assert np.array_equal(o4["grad_probs"], out["grad_probs"]), "grad_probs depends on p"
    # p = 0 gives zero outputs and gradients
    z = np.zeros_like(probs)
    assert np.all((orc.fwd(x, z, L) & 0x7FFF) == 0), "p=0 must give y = +-0"
    assert np.all((orc.bwd(x, z, gy, L)["grad_x"] & 0x7FFF) == 0), "p=0 must give grad_x = +-0"
    # thread count does not change bits
    o5 = orc.bwd(x, probs, gy, L, threads=7)
    o6 = orc.bwd(x, probs, gy, L, threads=1)
    assert np.array_equal(o5["grad_x"], o6["grad_x"]) and \
        np.array_equal(o5["grad_probs"], o6["grad_probs"]), "thread count changed bits"
    assert np.array_equal(orc.fwd(x, probs, L, threads=5), orc.fwd(x, probs, L, threads=1))


def pin_rows_n_used(orc):
    x, probs, gy, L = _small(seed=10, rows=40, inter=32)
    full_y = orc.fwd(x, probs, L)
    full = orc.bwd(x, probs, gy, L)
    for k in (0, 1, 17, 39, 40):
        for zp in (False, True):
            y = orc.fwd(x, probs, L, n_used=k, zero_padding=zp)
            o = orc.bwd(x, probs, gy, L, n_used=k, zero_padding=zp,
                        grad_probs_out=np.full(40, -3.5, dtype=np.float32))
            assert np.array_equal(y[:k], full_y[:k]), f"n_used={k}: live rows changed"
            assert np.array_equal(o["grad_x"][:k], full["grad_x"][:k])
            assert np.array_equal(o["grad_probs"][:k], full["grad_probs"][:k])
            pad = 0x0000 if zp else 0xFFFF
            assert np.all(y[k:] == pad) and np.all(o["grad_x"][k:] == pad), \
                f"n_used={k} zero_padding={zp}: padding rows wrong"
            assert np.all(o["grad_probs"][k:] == -3.5), "grad_probs written for a padding row"
    # out-of-range device counts are clamped
    assert np.all(orc.fwd(x, probs, L, n_used=-5, zero_padding=True) == 0)
    assert np.array_equal(orc.fwd(x, probs, L, n_used=1000), full_y)


def pin_rows_permutation(orc):
    x, probs, gy, L = _small(seed=11, rows=40, inter=32)
    perm = np.random.default_rng(3).permutation(40).astype(np.int32)
    # the map gathers the probability of each row and scatters its gradient
    y = orc.fwd(x, probs, L, permutation_map=perm)
    assert np.array_equal(y, orc.fwd(x, probs[perm], L)), "map must gather probs[map[r]]"
    o = orc.bwd(x, probs, gy, L, permutation_map=perm)
    ref = orc.bwd(x, probs[perm], gy, L)
    assert np.array_equal(o["grad_x"], ref["grad_x"])
    scattered = np.full(40, np.nan, dtype=np.float32)
    scattered[perm] = ref["grad_probs"]
    assert np.array_equal(o["grad_probs"], scattered), "map must scatter grad_probs[map[r]]"
    # with n_used, only the first n_used rows scatter
    o2 = orc.bwd(x, probs, gy, L, permutation_map=perm, n_used=25, zero_padding=True,
                 grad_probs_out=np.full(40, 9.0, dtype=np.float32))
    touched = np.zeros(40, dtype=bool)
    touched[perm[:25]] = True
    assert np.array_equal(o2["grad_probs"][touched], scattered[touched])
    assert np.all(o2["grad_probs"][~touched] == 9.0)
    assert np.all(o2["grad_x"][25:] == 0)


def pin_rows_dummy_entries(orc):
    x, probs, gy, L = _small(seed=12, rows=16, inter=16)
    perm = np.arange(16, dtype=np.int32)[::-1].copy()
    perm[3] = -1
    perm[7] = 16
    perm[9] = -2147483648
    for zp in (False, True):
        y = orc.fwd(x, probs, L, permutation_map=perm, zero_padding=zp)
        o = orc.bwd(x, probs, gy, L, permutation_map=perm, zero_padding=zp)
        pad = 0x0000 if zp else 0xFFFF
        for r in (3, 7, 9):
            assert np.all(y[r] == pad) and np.all(o["grad_x"][r] == pad), f"dummy row {r}"
        live = [r for r in range(16) if r not in (3, 7, 9)]
        ref = orc.fwd(x, probs[np.clip(perm, 0, 15)], L)
        assert np.array_equal(y[live], ref[live])
        untouched = np.setdiff1d(np.arange(16), perm[live])
        assert np.all(np.isnan(o["grad_probs"][untouched]))


ALL_PINS = [
    pin_rne_matches_torch,
    pin_unclamped_is_plain_swiglu,
    pin_probs_one_is_bare_activation,
    pin_fp32_path_matches_fp64_autograd,
    pin_inclusive_masks,
    pin_fp64_path_matches_autograd,
    pin_fp64_central_differences,
    pin_grad_probs_brute_force,
    pin_closed_forms,
    pin_structure,
    pin_rows_n_used,
    pin_rows_permutation,
    pin_rows_dummy_entries,
]
