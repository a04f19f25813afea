"""MoE elementwise operations: HIP path (through the C ABI) vs the MoE-ops oracle.

Bars: bitwise where the pages fix the result exactly (residual add = two unfused
adds; router-weight forward and grad_x = one fp32 product and one rounding;
squared ReLU forward and grad_x without the soft clamp; unpermute = a fixed-order
fp32 sum); within 1 bf16 ulp for the soft-clamped squared ReLU forward and
backward (tanh and sech^2 are evaluated by different fp32 formulas); grad_probs on
the row-scale criterion.
"""
import numpy as np
import pytest
import torch

import oracle.moe as moe_oracle
from bf16cmp import assert_within_ulp, grad_probs_violations
from memory_bound_elementwise_amd import (FusedMoEResidualAdd, RouterWeightMul, SquaredReluProbs,
                                          moe_residual_add, moe_router_weight_bwd,
                                          moe_router_weight_fwd, moe_squared_relu_probs_bwd,
                                          moe_squared_relu_probs_fwd, moe_unpermute_expert_order)
from memory_bound_elementwise_amd.moe_elementwise import load_library
from parity import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _rand(shape, dt, rng, scale=1.0, specials=True):
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    if specials and v.size >= 64:
        flat = v.reshape(-1)
        idx = rng.choice(flat.size, size=6 * max(1, flat.size // 500), replace=False)
        k = idx.size // 6
        flat[idx[:k]], flat[idx[k:2 * k]], flat[idx[2 * k:3 * k]] = np.inf, -np.inf, np.nan
        flat[idx[3 * k:4 * k]], flat[idx[4 * k:5 * k]] = 0.0, -0.0
        flat[idx[5 * k:]] = 65000.0 if dt == "f16" else 3e38
    t = torch.from_numpy(v).to(TD[dt])
    return t.numpy() if dt == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if dt != "f32" else np.ascontiguousarray(a))
    return (t if dt == "f32" else t.view(TD[dt])).to(DEV)


def _host(t, dt):
    t = t.cpu()
    return t.numpy() if dt == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def _same(a, b, dt):
    if dt == "f32":
        return np.array_equal(a.view(np.uint32), b.view(np.uint32)) or \
            bool(np.all((a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))))
    mant, expo = (0x7F, 0x7F80) if dt == "bf16" else (0x3FF, 0x7C00)
    na = ((a & expo) == expo) & ((a & mant) != 0)
    nb = ((b & expo) == expo) & ((b & mant) != 0)
    return bool(np.all((a == b) | (na & nb)))


def _same_by_rows(got, want, dt, what, block=4096):
    """_same over row blocks (bounds the temporaries at the full workload sizes)."""
    for r in range(0, got.shape[0], block):
        assert _same(got[r:r + block], want[r:r + block], dt), f"{what}: rows {r}..{r + block} differ"


def _within_ulp_by_rows(got, want, what, block=4096):
    for r in range(0, got.shape[0], block):
        assert_within_ulp(got[r:r + block], want[r:r + block], 1, f"{what} rows {r}..")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("n", [1, 7, 8, 1000, 4096 * 7 + 5, 1 << 22])
def test_residual_add(dt, n):
    rng = np.random.default_rng(n)
    e, s, r = _rand(n, dt, rng, 4.0), _rand(n, dt, rng, 4.0), _rand(n, dt, rng, 50.0)
    want = moe_oracle.get().residual_add(e, s, r, dt)
    out = torch.empty(n, dtype=TD[dt], device=DEV)
    moe_residual_add(_dev(e, dt), _dev(s, dt), _dev(r, dt), out)
    torch.cuda.synchronize()
    assert _same(_host(out, dt), want, dt), f"residual add {dt} n={n}"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_residual_add_in_place_and_grid(dt):
    rng = np.random.default_rng(5)
    n = 3 * 2048 * 61 + 3
    e, s, r = _rand(n, dt, rng), _rand(n, dt, rng), _rand(n, dt, rng, 10.0)
    want = moe_oracle.get().residual_add(e, s, r, dt)
    for nwg in (0, 1, 7, 1000):
        res = _dev(r, dt)
        moe_residual_add(_dev(e, dt), _dev(s, dt), res, res, num_workgroups=nwg)   # in place
        torch.cuda.synchronize()
        assert _same(_host(res, dt), want, dt), f"in place, {nwg} workgroups"


def test_residual_add_autograd():
    x = [torch.randn(64, 96, device=DEV, dtype=torch.bfloat16, requires_grad=True) for _ in range(3)]
    y = FusedMoEResidualAdd.apply(*x)
    ref = x[2].detach() + (x[0].detach() + x[1].detach())
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    g = torch.randn_like(y)
    y.backward(g)
    assert all(torch.equal(t.grad, g) for t in x)


def test_residual_add_full_size():
    """6720 x 7168 bf16 (the MoE workload), default launch: every element, bitwise."""
    from memory_bound_elementwise_amd.workloads import make_moe_inputs
    inp = make_moe_inputs("residual_add", seed=0)
    e, sh, r = inp["expert"], inp["shared"], inp["residual"]
    say(f"[residual add full] {e.shape[0]}x{e.shape[1]}")
    out = torch.empty(e.shape, dtype=torch.bfloat16, device=DEV)
    moe_residual_add(_dev(e, "bf16"), _dev(sh, "bf16"), _dev(r, "bf16"), out)
    torch.cuda.synchronize()
    want = moe_oracle.get().residual_add(e, sh, r, "bf16")
    assert _same(_host(out, "bf16"), want, "bf16")


# ---------------------------------------------------------------------------
ROUTER_TYPES = [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f16", "f32"), ("f32", "f32")]


@pytest.mark.parametrize("x_dt,out_dt", ROUTER_TYPES)
@pytest.mark.parametrize("tokens,hidden", [(1, 8), (333, 520), (1027, 2048), (64, 7168 + 8), (96, 7168)])
def test_router_weight(x_dt, out_dt, tokens, hidden):
    """7168 columns: the backward's waves take quarter rows (one masked chunk each)."""
    rng = np.random.default_rng(tokens + hidden)
    x = _rand((tokens, hidden), x_dt, rng, 3.0, specials=False)
    g = _rand((tokens, hidden), out_dt, rng, 1.0, specials=False)
    p = rng.uniform(0, 1, tokens).astype(np.float32)
    orc = moe_oracle.get()
    out = torch.empty((tokens, hidden), dtype=TD[out_dt], device=DEV)
    dp = torch.from_numpy(p).to(DEV)
    moe_router_weight_fwd(_dev(x, x_dt), dp, out)
    gx = torch.empty((tokens, hidden), dtype=TD[x_dt], device=DEV)
    gp = torch.full((tokens,), -7.0, device=DEV)
    moe_router_weight_bwd(_dev(g, out_dt), _dev(x, x_dt), dp, gx, gp)
    torch.cuda.synchronize()
    assert _same(_host(out, out_dt), orc.router_weight_fwd(x, x_dt, p, out_dt), out_dt), "router fwd"
    ref = orc.router_weight_bwd(g, out_dt, x, x_dt, p)
    assert _same(_host(gx, x_dt), ref["grad_x"], x_dt), "router grad_x"
    bad = grad_probs_violations(gp.cpu().numpy(), ref["grad_probs_f64"], ref["row_scale"])
    assert bad.size == 0, f"router grad_probs: {bad.size} rows off"


@pytest.mark.parametrize("hidden", [5120, 7168, 8192])
def test_router_weight_rows_split_over_waves(hidden):
    """Rows of 4 or more column chunks are shared by a workgroup's four waves (5, 7 and 4
    chunks here). The forward splits the chunks; where they do not divide by four (5120,
    7168) the backward's waves take quarter rows instead. The probability gradient adds
    the waves' partials in wave order, so every grid gives the same bits; outputs
    requested alone take the same paths."""
    rng = np.random.default_rng(hidden)
    tokens = 777
    x = _rand((tokens, hidden), "bf16", rng, 3.0, specials=False)
    g = _rand((tokens, hidden), "bf16", rng, 1.0, specials=False)
    p = rng.uniform(0, 1, tokens).astype(np.float32)
    orc = moe_oracle.get()
    ref = orc.router_weight_bwd(g, "bf16", x, "bf16", p)
    want_y = orc.router_weight_fwd(x, "bf16", p, "bf16")
    xd, gd, dp = _dev(x, "bf16"), _dev(g, "bf16"), torch.from_numpy(p).to(DEV)
    first = None
    for nwg in (0, 1, 2, 3, 777, 1024):
        y = torch.empty((tokens, hidden), dtype=torch.bfloat16, device=DEV)
        gx = torch.empty_like(y)
        gp = torch.full((tokens,), -7.0, device=DEV)
        moe_router_weight_fwd(xd, dp, y, num_workgroups=nwg)
        moe_router_weight_bwd(gd, xd, dp, gx, gp, num_workgroups=nwg)
        torch.cuda.synchronize()
        got = (_host(y, "bf16"), _host(gx, "bf16"), gp.cpu().numpy())
        if first is None:
            first = got
            assert _same(got[0], want_y, "bf16") and _same(got[1], ref["grad_x"], "bf16")
            assert grad_probs_violations(got[2], ref["grad_probs_f64"], ref["row_scale"]).size == 0
        else:
            assert np.array_equal(got[0], first[0]) and np.array_equal(got[1], first[1]), f"grid {nwg}"
            assert np.array_equal(got[2].view(np.uint32), first[2].view(np.uint32)), f"grid {nwg}: grad_probs bits"
    gp_only = torch.empty(tokens, device=DEV)
    moe_router_weight_bwd(gd, xd, dp, None, gp_only)
    gx_only = torch.empty((tokens, hidden), dtype=torch.bfloat16, device=DEV)
    moe_router_weight_bwd(gd, None, dp, gx_only, None, x_dtype="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(gp_only.cpu().numpy().view(np.uint32), first[2].view(np.uint32))
    assert np.array_equal(_host(gx_only, "bf16"), first[1])


def test_router_weight_optional_outputs():
    rng = np.random.default_rng(9)
    x = _rand((100, 512), "bf16", rng, specials=False)
    g = _rand((100, 512), "bf16", rng, specials=False)
    p = torch.from_numpy(rng.uniform(0, 1, 100).astype(np.float32)).to(DEV)
    ref = moe_oracle.get().router_weight_bwd(g, "bf16", x, "bf16", p.cpu().numpy())
    gx = torch.empty((100, 512), dtype=torch.bfloat16, device=DEV)
    moe_router_weight_bwd(_dev(g, "bf16"), None, p, gx, None, x_dtype="bf16")   # x not needed
    gp = torch.empty(100, device=DEV)
    moe_router_weight_bwd(_dev(g, "bf16"), _dev(x, "bf16"), p, None, gp)
    torch.cuda.synchronize()
    assert _same(_host(gx, "bf16"), ref["grad_x"], "bf16")
    assert grad_probs_violations(gp.cpu().numpy(), ref["grad_probs_f64"], ref["row_scale"]).size == 0


def test_router_weight_autograd_and_grid():
    x = torch.randn(300, 1024, device=DEV, dtype=torch.bfloat16, requires_grad=True)
    p = torch.rand(300, 1, device=DEV, requires_grad=True)
    y = RouterWeightMul.apply(x, p, torch.bfloat16)
    assert torch.equal(y.view(torch.int16), (x.detach().float() * p.detach()).to(torch.bfloat16).view(torch.int16))
    g = torch.randn_like(y)
    y.backward(g)
    assert torch.equal(x.grad.view(torch.int16), (g.float() * p.detach()).to(torch.bfloat16).view(torch.int16))
    exact = (g.double() * x.detach().double()).sum(-1)
    scale = (g.double() * x.detach().double()).abs().sum(-1)
    assert torch.all((p.grad.reshape(-1).double() - exact).abs() <= 1e-6 + 1e-5 * scale)
    outs = []
    for nwg in (0, 1, 5, 999):
        o = torch.empty(300, 1024, device=DEV)
        gp = torch.empty(300, device=DEV)
        moe_router_weight_fwd(x.detach(), p.detach().reshape(-1), o, num_workgroups=nwg)
        moe_router_weight_bwd(g, x.detach(), p.detach().reshape(-1), None, gp, num_workgroups=nwg)
        outs.append((o.clone(), gp.clone()))
    for o, gp in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(gp.view(torch.int32), outs[0][1].view(torch.int32))


def test_router_weight_full_size():
    """53760 x 7168 bf16 (the MoE workload), default launch (the backward's waves take
    quarter rows): every row against the oracle, forward and grad_x bitwise, every
    grad_probs row on the row-scale criterion."""
    from memory_bound_elementwise_amd.workloads import make_moe_inputs
    inp = make_moe_inputs("router_weight", seed=0)
    x, p, g = inp["x"], inp["probs"], inp["grad_out"]
    tokens, hidden = x.shape
    say(f"[router full] {tokens}x{hidden}")
    xd, gd, dp = _dev(x, "bf16"), _dev(g, "bf16"), torch.from_numpy(p).to(DEV)
    out = torch.empty_like(xd)
    gx = torch.empty_like(xd)
    gp = torch.full((tokens,), -7.0, device=DEV)
    moe_router_weight_fwd(xd, dp, out)
    moe_router_weight_bwd(gd, xd, dp, gx, gp)
    torch.cuda.synchronize()
    orc = moe_oracle.get()
    _same_by_rows(_host(out, "bf16"), orc.router_weight_fwd(x, "bf16", p, "bf16"), "bf16", "router fwd")
    del out
    ref = orc.router_weight_bwd(g, "bf16", x, "bf16", p)
    _same_by_rows(_host(gx, "bf16"), ref["grad_x"], "bf16", "router grad_x")
    bad = grad_probs_violations(gp.cpu().numpy(), ref["grad_probs_f64"], ref["row_scale"])
    assert bad.size == 0, f"router grad_probs: {bad.size} rows off"


# ---------------------------------------------------------------------------
def _sq_run(x, p, **kw):
    rows, hidden = x.shape
    y = torch.full((rows, hidden), -1, dtype=torch.int16, device=DEV)
    nu = kw.pop("n_used", None)
    pm = kw.pop("permutation_map", None)
    moe_squared_relu_probs_fwd(_dev(x, "bf16").view(torch.int16), torch.from_numpy(p).to(DEV), y,
                               n_used=None if nu is None else torch.tensor([nu], dtype=torch.int32, device=DEV),
                               permutation_map=None if pm is None else torch.from_numpy(pm).to(DEV), **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("clamp_scale", [None, 0.5, 4.0, 30.0])
@pytest.mark.parametrize("rows,hidden", [(7, 8), (513, 1536), (2000, 2048 + 8)])
def test_squared_relu(clamp_scale, rows, hidden):
    rng = np.random.default_rng(rows)
    x = _rand((rows, hidden), "bf16", rng, 6.0)
    p = rng.uniform(0, 1, rows).astype(np.float32)
    got = _sq_run(x, p, clamp_scale=clamp_scale)
    want = moe_oracle.get().squared_relu_probs(x, p, clamp_scale=clamp_scale)
    if clamp_scale is None:
        assert _same(got, want, "bf16"), "squared relu without clamp must be bit-exact"
    else:
        assert_within_ulp(got, want, 1, f"soft clamp s={clamp_scale}")


@pytest.mark.parametrize("clamp_scale", [None, 1.0, 8.0])
def test_squared_relu_every_bf16_pattern(clamp_scale):
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    p = np.linspace(0.05, 1.0, 256).astype(np.float32)
    got = _sq_run(x, p, clamp_scale=clamp_scale)
    want = moe_oracle.get().squared_relu_probs(x, p, clamp_scale=clamp_scale)
    if clamp_scale is None:
        assert _same(got, want, "bf16")
    else:
        assert_within_ulp(got, want, 1, f"sweep s={clamp_scale}")


@pytest.mark.parametrize("zero_padding", [False, True])
def test_squared_relu_rows(zero_padding):
    rng = np.random.default_rng(11)
    rows, hidden = 4096, 1024
    x = _rand((rows, hidden), "bf16", rng, 3.0, specials=False)
    p = rng.uniform(0, 1, rows).astype(np.float32)
    pm = rng.permutation(rows).astype(np.int32)
    pm[rng.choice(rows, 40, replace=False)] = -1
    for n_used in (0, 1, 3000, rows, rows + 9, -4):
        kw = dict(clamp_scale=2.0, n_used=n_used, permutation_map=pm, zero_padding=zero_padding)
        got = _sq_run(x, p, **kw)
        want = moe_oracle.get().squared_relu_probs(x, p, **kw)
        assert_within_ulp(got, want, 1, f"rows n_used={n_used}")
        assert np.array_equal(got == 0xFFFF, want == 0xFFFF)


@pytest.mark.parametrize("clamp_scale", [None, 4.0])
def test_squared_relu_full_size(clamp_scale):
    """53,760 x 2,048 (the MoE workload), default launch; every row against the oracle."""
    from memory_bound_elementwise_amd.workloads import make_moe_inputs
    inp = make_moe_inputs("squared_relu", seed=0)
    x, p = inp["x"], inp["probs"]
    rows, hidden = x.shape
    say(f"[sqrelu fwd full] s={clamp_scale} {rows}x{hidden}")
    y = torch.empty((rows, hidden), dtype=torch.bfloat16, device=DEV)
    moe_squared_relu_probs_fwd(_dev(x, "bf16"), torch.from_numpy(p).to(DEV), y, clamp_scale=clamp_scale)
    torch.cuda.synchronize()
    got = _host(y, "bf16")
    want = moe_oracle.get().squared_relu_probs(x, p, clamp_scale=clamp_scale)
    if clamp_scale is None:
        _same_by_rows(got, want, "bf16", "full size")
    else:
        _within_ulp_by_rows(got, want, "full size")


# ---------------------------------------------------------------------------
GP_SENTINEL = -12345.5


def _sqb_run(x, p, g, with_gp=True, **kw):
    rows, hidden = x.shape
    gx = torch.full((rows, hidden), -1, dtype=torch.int16, device=DEV)
    gp = torch.full((rows,), GP_SENTINEL, dtype=torch.float32, device=DEV) if with_gp else None
    nu = kw.pop("n_used", None)
    pm = kw.pop("permutation_map", None)
    moe_squared_relu_probs_bwd(_dev(x, "bf16").view(torch.int16), torch.from_numpy(p).to(DEV),
                               _dev(g, "bf16").view(torch.int16), gx, gp,
                               n_used=None if nu is None else torch.tensor([nu], dtype=torch.int32, device=DEV),
                               permutation_map=None if pm is None else torch.from_numpy(pm).to(DEV), **kw)
    torch.cuda.synchronize()
    return gx.cpu().numpy().view(np.uint16), (None if gp is None else gp.cpu().numpy())


FLT_MAX = float(np.finfo(np.float32).max)


def _check_grad_probs(got, want, what):
    """Rows on the row-scale criterion; rows holding inf / NaN terms must agree in kind
    (NaN, or the same infinity). Rows whose |terms| add up past the fp32 range are not
    compared: an fp32 sum may overflow there whatever its order."""
    scale = want["row_scale"]
    fin = np.isfinite(want["grad_probs_f64"]) & np.isfinite(scale)
    ok = fin & (scale < FLT_MAX)
    bad = grad_probs_violations(got[ok], want["grad_probs_f64"][ok], scale[ok])
    assert bad.size == 0, f"{what}: grad_probs off on {bad.size} rows"
    w = want["grad_probs"][~fin]
    gg = got[~fin]
    assert np.array_equal(np.isnan(gg), np.isnan(w)) and np.array_equal(gg[np.isinf(w)], w[np.isinf(w)]), \
        f"{what}: non-finite grad_probs differ"


def _check_sqb(gx, gp, want, clamp_scale, what):
    if clamp_scale is None:
        assert _same(gx, want["grad_x"], "bf16"), f"{what}: grad_x without clamp must be bit-exact"
    else:
        assert_within_ulp(gx, want["grad_x"], 1, what)
    if gp is not None:
        _check_grad_probs(gp, want, what)


@pytest.mark.parametrize("clamp_scale", [None, 0.5, 4.0, 30.0])
@pytest.mark.parametrize("rows,hidden", [(7, 8), (513, 1536), (2000, 2048 + 8)])
def test_squared_relu_bwd(clamp_scale, rows, hidden):
    rng = np.random.default_rng(rows + 17)
    x = _rand((rows, hidden), "bf16", rng, 6.0)
    g = _rand((rows, hidden), "bf16", rng, 1.0, specials=rows != 2000)
    p = rng.uniform(0, 1, rows).astype(np.float32)
    gx, gp = _sqb_run(x, p, g, clamp_scale=clamp_scale)
    want = moe_oracle.get().squared_relu_probs_bwd(x, p, g, clamp_scale=clamp_scale)
    _check_sqb(gx, gp, want, clamp_scale, f"bwd s={clamp_scale} {rows}x{hidden}")


@pytest.mark.parametrize("clamp_scale", [None, 1.0, 8.0])
@pytest.mark.parametrize("sweep", ["x", "grad_y"])
def test_squared_relu_bwd_every_bf16_pattern(clamp_scale, sweep):
    """All 65,536 bf16 patterns of x (grad_y ~ N(0,1)), or of grad_y (x fixed per row)."""
    rng = np.random.default_rng(5)
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    other = _rand((256, 256), "bf16", rng, 2.0, specials=False)
    x, g = (every, other) if sweep == "x" else (other, every)
    p = np.linspace(0.05, 1.0, 256).astype(np.float32)
    gx, gp = _sqb_run(x, p, g, clamp_scale=clamp_scale)
    want = moe_oracle.get().squared_relu_probs_bwd(x, p, g, clamp_scale=clamp_scale)
    _check_sqb(gx, gp, want, clamp_scale, f"sweep {sweep} s={clamp_scale}")


@pytest.mark.parametrize("zero_padding", [False, True])
def test_squared_relu_bwd_rows(zero_padding):
    rng = np.random.default_rng(12)
    rows, hidden = 4096, 1024
    x = _rand((rows, hidden), "bf16", rng, 3.0, specials=False)
    g = _rand((rows, hidden), "bf16", rng, 1.0, specials=False)
    p = rng.uniform(0, 1, rows).astype(np.float32)
    pm = rng.permutation(rows).astype(np.int32)
    pm[rng.choice(rows, 40, replace=False)] = -1
    for clamp_scale in (None, 2.0):
        for n_used in (0, 1, 3000, rows, rows + 9, -4):
            kw = dict(clamp_scale=clamp_scale, n_used=n_used, permutation_map=pm, zero_padding=zero_padding)
            gx, gp = _sqb_run(x, p, g, **kw)
            want = moe_oracle.get().squared_relu_probs_bwd(x, p, g, **kw)
            assert np.array_equal(gx == 0xFFFF, want["grad_x"] == 0xFFFF), f"untouched rows n_used={n_used}"
            assert np.array_equal(gp == GP_SENTINEL, want["grad_probs"] == GP_SENTINEL), \
                f"untouched grad_probs slots n_used={n_used}"
            live = want["grad_probs"] != GP_SENTINEL
            if clamp_scale is None:
                assert _same(gx, want["grad_x"], "bf16")
            else:
                assert_within_ulp(gx, want["grad_x"], 1, f"rows n_used={n_used}")
            bad = grad_probs_violations(gp[live], want["grad_probs_f64"][live], want["row_scale"][live])
            assert bad.size == 0
    # without grad_probs only grad_x is written
    gx, _ = _sqb_run(x, p, g, with_gp=False, clamp_scale=2.0)
    assert_within_ulp(gx, moe_oracle.get().squared_relu_probs_bwd(x, p, g, clamp_scale=2.0)["grad_x"], 1, "no gp")


def test_squared_relu_bwd_grid_invariant():
    """grad_x and grad_probs bits do not depend on the workgroup count, run to run."""
    rng = np.random.default_rng(13)
    rows, hidden = 3001, 2048
    x = _rand((rows, hidden), "bf16", rng, 3.0, specials=False)
    g = _rand((rows, hidden), "bf16", rng, 1.0, specials=False)
    p = rng.uniform(0, 1, rows).astype(np.float32)
    for s in (None, 4.0):
        ref = None
        for nwg in (0, 1, 37, 256, 1024, 0):
            gx, gp = _sqb_run(x, p, g, clamp_scale=s, num_workgroups=nwg)
            if ref is None:
                ref = (gx, gp)
                _check_sqb(gx, gp, moe_oracle.get().squared_relu_probs_bwd(x, p, g, clamp_scale=s), s, "grid")
            else:
                assert np.array_equal(gx, ref[0]) and np.array_equal(gp.view(np.uint32), ref[1].view(np.uint32)), \
                    f"grid {nwg} changed bits (s={s})"


@pytest.mark.parametrize("clamp_scale", [None, 4.0])
def test_squared_relu_autograd(clamp_scale):
    rng = np.random.default_rng(14)
    rows, hidden = 300, 512
    x = _rand((rows, hidden), "bf16", rng, 3.0, specials=False)
    g = _rand((rows, hidden), "bf16", rng, 1.0, specials=False)
    p = rng.uniform(0, 1, (rows, 1)).astype(np.float32)
    tx = _dev(x, "bf16").requires_grad_(True)
    tp = torch.from_numpy(p).to(DEV).requires_grad_(True)
    y = SquaredReluProbs.apply(tx, tp, clamp_scale)
    y.backward(_dev(g, "bf16"))
    orc = moe_oracle.get()
    assert_within_ulp(_host(y.detach(), "bf16"), orc.squared_relu_probs(x, p, clamp_scale=clamp_scale), 1, "fwd")
    want = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=clamp_scale)
    _check_sqb(_host(tx.grad, "bf16"), tp.grad.reshape(-1).cpu().numpy(), want, clamp_scale, "autograd")
    assert tp.grad.shape == tp.shape


@pytest.mark.parametrize("clamp_scale", [None, 4.0])
def test_squared_relu_bwd_full_size(clamp_scale):
    """53,760 x 2,048 (the MoE workload), default launch; every row against the oracle."""
    from memory_bound_elementwise_amd.workloads import make_moe_inputs
    inp = make_moe_inputs("squared_relu", seed=0)
    x, p, gys = inp["x"], inp["probs"], inp["grad_y"]
    rows, hidden = x.shape
    gy = _dev(gys, "bf16")
    xd = _dev(x, "bf16")
    gx = torch.empty_like(xd)
    gp = torch.full((rows,), GP_SENTINEL, device=DEV)
    say(f"[sqrelu bwd full] s={clamp_scale} {rows}x{hidden}")
    moe_squared_relu_probs_bwd(xd, torch.from_numpy(p).to(DEV), gy, gx, gp, clamp_scale=clamp_scale)
    torch.cuda.synchronize()
    want = moe_oracle.get().squared_relu_probs_bwd(x, p, gys, clamp_scale=clamp_scale)
    got = _host(gx, "bf16")
    if clamp_scale is None:
        _same_by_rows(got, want["grad_x"], "bf16", "full size grad_x")
    else:
        _within_ulp_by_rows(got, want["grad_x"], "full size grad_x")
    _check_grad_probs(gp.cpu().numpy(), want, "full size")


# ---------------------------------------------------------------------------
def _unpermute_inputs(rng, tokens, E, hidden, density):
    valid = rng.random((tokens, E)) < density
    # rows grouped by expert (the grouped GEMM's order), tokens in order within each
    im = np.full((tokens, E), -1, np.int32)
    row = 0
    for e in range(E):
        ts = np.flatnonzero(valid[:, e])
        im[ts, e] = np.arange(row, row + ts.size)
        row += ts.size
    eo = _rand((max(row, 1), hidden), "bf16", rng, 1.0, specials=False)
    return eo, im


@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
@pytest.mark.parametrize("tokens,E,hidden", [(1, 1, 8), (300, 4, 520), (2048, 8, 2048), (129, 70, 64),
                                             (64, 300, 16)])
def test_unpermute(out_dt, tokens, E, hidden):
    rng = np.random.default_rng(tokens * E)
    eo, im = _unpermute_inputs(rng, tokens, E, hidden, 0.5)
    im[0, 0] = eo.shape[0] + 3        # an out-of-range entry contributes nothing
    want = moe_oracle.get().unpermute(eo, im, out_dt)
    out = torch.empty((tokens, hidden), dtype=TD[out_dt], device=DEV)
    moe_unpermute_expert_order(_dev(eo, "bf16"), torch.from_numpy(im).to(DEV), out)
    torch.cuda.synchronize()
    assert _same(_host(out, out_dt), want, out_dt), "unpermute must be bit-exact (fixed order)"


@pytest.mark.parametrize("E", [2, 3, 5, 6, 7])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_unpermute_experts_below_group(E, out_dt):
    """Expert counts that leave part of the 4- or 8-wide gather group empty."""
    rng = np.random.default_rng(100 + E)
    tokens, hidden = 777, 1032
    eo, im = _unpermute_inputs(rng, tokens, E, hidden, 0.6)
    want = moe_oracle.get().unpermute(eo, im, out_dt)
    out = torch.empty((tokens, hidden), dtype=TD[out_dt], device=DEV)
    moe_unpermute_expert_order(_dev(eo, "bf16"), torch.from_numpy(im).to(DEV), out)
    torch.cuda.synchronize()
    assert _same(_host(out, out_dt), want, out_dt)


@pytest.mark.parametrize("E", [4, 8, 12])
def test_unpermute_grid_invariant(E):
    """Same bits for any workgroup count, including one workgroup (every wave walks
    hundreds of tokens and reloads its map rows many times)."""
    rng = np.random.default_rng(200 + E)
    tokens, hidden = 2048, 520
    eo, im = _unpermute_inputs(rng, tokens, E, hidden, 0.5)
    want = moe_oracle.get().unpermute(eo, im, "f32")
    eod, imd = _dev(eo, "bf16"), torch.from_numpy(im).to(DEV)
    vt = torch.tensor([tokens - 5], dtype=torch.int32, device=DEV)
    for nwg in (1, 3, 240, 256, 1024, 0):
        out = torch.full((tokens, hidden), float("nan"), device=DEV)
        moe_unpermute_expert_order(eod, imd, out, valid_tokens=vt, num_workgroups=nwg)
        torch.cuda.synchronize()
        o = _host(out, "f32")
        assert _same(o[:tokens - 5], want[:tokens - 5], "f32"), f"grid {nwg}"
        assert np.all(np.isnan(o[tokens - 5:])), f"grid {nwg}: tokens past the bound written"


@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_unpermute_full_size(out_dt):
    """6720 tokens x 8 local experts x 7168 (the MoE workload), default launch; every
    token against the oracle, bitwise."""
    from memory_bound_elementwise_amd.workloads import make_moe_inputs
    inp = make_moe_inputs("unpermute", seed=0)
    eo, im = inp["expert_output"], inp["inverse_map"]
    tokens, hidden = im.shape[0], eo.shape[1]
    say(f"[unpermute full] {tokens}x{im.shape[1]}x{hidden} {out_dt}")
    out = torch.empty((tokens, hidden), dtype=TD[out_dt], device=DEV)
    moe_unpermute_expert_order(_dev(eo, "bf16"), torch.from_numpy(im).to(DEV), out)
    torch.cuda.synchronize()
    want = moe_oracle.get().unpermute(eo, im, out_dt)
    _same_by_rows(_host(out, out_dt), want, out_dt, "unpermute")


def test_unpermute_order_and_bound():
    hidden = 64
    big = np.zeros((3, hidden), np.uint16)
    big[0], big[1], big[2] = 0x4B80, 0x3F80, 0xCB80          # 2^24, 1, -2^24
    im = np.array([[0, 1, 2], [2, 1, 0], [1, -1, -1], [0, 2, 1]], np.int32)
    out = torch.full((4, hidden), float("nan"), device=DEV)
    vt = torch.tensor([3], dtype=torch.int32, device=DEV)
    moe_unpermute_expert_order(_dev(big, "bf16"), torch.from_numpy(im).to(DEV), out, valid_tokens=vt)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[0] == 0.0) and np.all(o[1] == 1.0) and np.all(o[2] == 1.0)
    assert np.all(np.isnan(o[3])), "token at valid_tokens must not be written"


def test_moe_error_paths():
    lib = load_library()
    a = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    assert lib.moe_residual_add(a.data_ptr() + 2, a.data_ptr(), a.data_ptr(), a.data_ptr(), 8, 0, None, 0) == 2
    say("[moe] error paths ok")


def test_widest_rows():
    """hidden = 2^26, the widest row the MoE C ABI accepts (an fp32 row is 2^28 bytes):
    router weight forward and backward in fp32, the soft-clamped squared ReLU forward and
    backward, and the unpermute with fp32 output, on two rows or tokens each; every
    element against the oracle."""
    H = 1 << 26
    rng = np.random.default_rng(26)
    orc = moe_oracle.get()
    say(f"[moe widest] router fp32, 2 x {H}")
    x = _rand((2, H), "f32", rng, 3.0, specials=False)
    g = _rand((2, H), "f32", rng, 1.0, specials=False)
    p = rng.uniform(0, 1, 2).astype(np.float32)
    dp = torch.from_numpy(p).to(DEV)
    xd, gd = _dev(x, "f32"), _dev(g, "f32")
    out = torch.empty((2, H), dtype=torch.float32, device=DEV)
    gx = torch.empty_like(out)
    gp = torch.full((2,), -7.0, device=DEV)
    moe_router_weight_fwd(xd, dp, out)
    moe_router_weight_bwd(gd, xd, dp, gx, gp)
    torch.cuda.synchronize()
    assert _same(_host(out, "f32"), orc.router_weight_fwd(x, "f32", p, "f32"), "f32"), "router fwd"
    ref = orc.router_weight_bwd(g, "f32", x, "f32", p)
    assert _same(_host(gx, "f32"), ref["grad_x"], "f32"), "router grad_x"
    assert grad_probs_violations(gp.cpu().numpy(), ref["grad_probs_f64"], ref["row_scale"]).size == 0
    del x, g, xd, gd, out, gx, ref

    say(f"[moe widest] squared ReLU, 2 x {H}")
    xb = _rand((2, H), "bf16", rng, 6.0, specials=False)
    gb = _rand((2, H), "bf16", rng, 1.0, specials=False)
    xbd = _dev(xb, "bf16")
    yq = torch.empty_like(xbd)
    moe_squared_relu_probs_fwd(xbd, dp, yq, clamp_scale=4.0)
    torch.cuda.synchronize()
    assert_within_ulp(_host(yq, "bf16"), orc.squared_relu_probs(xb, p, clamp_scale=4.0), 1, "sqrelu fwd")
    gxq = torch.empty_like(xbd)
    gpq = torch.full((2,), GP_SENTINEL, device=DEV)
    moe_squared_relu_probs_bwd(xbd, dp, _dev(gb, "bf16"), gxq, gpq, clamp_scale=4.0)
    torch.cuda.synchronize()
    _check_sqb(_host(gxq, "bf16"), gpq.cpu().numpy(),
               orc.squared_relu_probs_bwd(xb, p, gb, clamp_scale=4.0), 4.0, "sqrelu widest")
    del xb, gb, xbd, yq, gxq

    say(f"[moe widest] unpermute fp32, 2 tokens x 2 experts x {H}")
    eo = _rand((3, H), "bf16", rng, 1.0, specials=False)
    im = np.array([[0, 1], [2, -1]], np.int32)
    uo = torch.empty((2, H), dtype=torch.float32, device=DEV)
    moe_unpermute_expert_order(_dev(eo, "bf16"), torch.from_numpy(im).to(DEV), uo)
    torch.cuda.synchronize()
    assert _same(_host(uo, "f32"), orc.unpermute(eo, im, "f32"), "f32"), "unpermute"
    say("[moe widest] ok")
