"""Pins of the MoE-ops oracle (``oracle/moe.py``) against values fixed independently.

Each ``pin_*`` takes a ``MoeOracle`` and raises ``AssertionError`` on disagreement.

* fp16 conversions     -> pin_f16_conversions (numpy's float16 casts, every pattern)
* residual add         -> pin_residual_add (torch CPU: residual + (expert + shared) in
                          the same dtype, i.e. the two unfused adds, bitwise)
* router weight fwd    -> pin_router_weight_fwd (torch (x.float() * p).to(dtype), bitwise)
* router weight bwd    -> pin_router_weight_bwd (torch fp32 autograd of that expression:
                          grad_x bitwise, grad_probs on the row-scale criterion; fp64 sums)
* squared ReLU         -> pin_squared_relu_no_clamp (torch bf16 relu(x)**2, then * p,
                          bitwise), pin_squared_relu_clamp (torch fp64 reference within
                          1 ulp; large scale reduces to the unclamped fp32 square),
                          pin_squared_relu_rows (n_used / map / padding rules)
* squared ReLU bwd     -> pin_squared_relu_bwd_fd (central differences of the fp64 forward
                          for grad_x and grad_probs, out to tanh's saturation),
                          pin_squared_relu_bwd_structure (s -> inf reduces to the unclamped
                          gradient; linear in g; grad_probs free of p and equal to the
                          forward's output at p = 1 without the clamp; masks and special
                          values), pin_squared_relu_bwd_rows (n_used / map / padding)
* unpermute            -> pin_unpermute (numpy float32 running sums in expert order;
                          single-contribution tokens copy the row exactly; bounds)
* row threads          -> pin_thread_count_invariance (every op, 1 thread against several:
                          the same bits, padding and untouched slots included)
"""
from __future__ import annotations

import math

import numpy as np
import torch

from bf16cmp import assert_within_ulp, bf16_bits_to_f32, grad_probs_violations

DT_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _np_to_torch(a: np.ndarray, dt: str) -> torch.Tensor:
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(DT_TORCH[dt])


def _torch_to_np(t: torch.Tensor, dt: str) -> np.ndarray:
    if dt == "f32":
        return t.to(torch.float32).numpy()
    return t.to(DT_TORCH[dt]).view(torch.int16).numpy().view(np.uint16)


def _draw(shape, dt, rng, scale=1.0, specials=True):
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    if specials:
        flat = v.reshape(-1)
        k = max(1, flat.size // 200)
        idx = rng.choice(flat.size, size=k * 6, replace=False)
        flat[idx[:k]] = np.inf
        flat[idx[k:2 * k]] = -np.inf
        flat[idx[2 * k:3 * k]] = np.nan
        flat[idx[3 * k:4 * k]] = 0.0
        flat[idx[4 * k:5 * k]] = -0.0
        flat[idx[5 * k:]] = 1e-41 if dt != "f16" else 3e-6
    return _torch_to_np(torch.from_numpy(v), dt)


def _same_bits(a: np.ndarray, b: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        an, bn = np.isnan(a), np.isnan(b)
        return (a.view(np.uint32) == b.view(np.uint32)) | (an & bn)
    aexp = (a & 0x7F80) == 0x7F80 if dt == "bf16" else (a & 0x7C00) == 0x7C00
    bexp = (b & 0x7F80) == 0x7F80 if dt == "bf16" else (b & 0x7C00) == 0x7C00
    mant = 0x7F if dt == "bf16" else 0x3FF
    an = aexp & ((a & mant) != 0)
    bn = bexp & ((b & mant) != 0)
    return (a == b) | (an & bn)


def pin_f16_conversions(orc):
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f32_from_f16(allp)
    want = allp.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)), "fp16 -> fp32"
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # fp32 values on and around fp16 rounding boundaries, incl. the subnormal range
    halves = (allp.view(np.float16).astype(np.float32))
    fin = np.isfinite(halves)
    mids = ((halves[fin][:-1].astype(np.float64) + halves[fin][1:]) / 2).astype(np.float32)
    f = np.concatenate([bits.view(np.float32), mids, np.nextafter(mids, np.inf),
                        np.nextafter(mids, -np.inf), np.float32([65504, 65519.99, 65520, 65536, 1e9])])
    got = orc.f16_from_f32(f)
    with np.errstate(over="ignore"):
        want = f.astype(np.float16).view(np.uint16)
    ok = _same_bits(got, want, "f16")
    assert ok.all(), f"fp32 -> fp16 differs at {np.flatnonzero(~ok)[:5]} ({f[~ok][:5]})"


def pin_residual_add(orc):
    rng = np.random.default_rng(1)
    for dt in ("bf16", "f16", "f32"):
        n = 1 << 18
        e = _draw(n, dt, rng, 4.0)
        s = _draw(n, dt, rng, 4.0)
        r = _draw(n, dt, rng, 100.0)
        got = orc.residual_add(e, s, r, dt)
        te, ts, tr = (_np_to_torch(v, dt) for v in (e, s, r))
        want = _torch_to_np(tr + (te + ts), dt)
        ok = _same_bits(got, want, dt)
        assert ok.all(), f"residual add {dt}: {int((~ok).sum())} mismatches"
        # the inner sum is rounded to the dtype before the residual add: for 16-bit
        # types a single fp32 sum of all three differs somewhere
        if dt != "f32":
            one = _torch_to_np((tr.float() + (te.float() + ts.float())).to(DT_TORCH[dt]), dt)
            assert not _same_bits(got, one, dt).all(), "inner rounding not observable"


def pin_router_weight_fwd(orc):
    rng = np.random.default_rng(2)
    for x_dt in ("bf16", "f16", "f32"):
        for out_dt in sorted({x_dt, "f32"}):
            x = _draw((64, 96), x_dt, rng, 3.0)
            p = rng.uniform(0, 1, 64).astype(np.float32)
            p[3] = 0.0
            got = orc.router_weight_fwd(x, x_dt, p, out_dt)
            want = _torch_to_np((_np_to_torch(x, x_dt).float() * torch.from_numpy(p)[:, None])
                                .to(DT_TORCH[out_dt]), out_dt)
            assert _same_bits(got, want, out_dt).all(), f"router fwd {x_dt}->{out_dt}"


def pin_router_weight_bwd(orc):
    rng = np.random.default_rng(3)
    for x_dt in ("bf16", "f16", "f32"):
        for out_dt in sorted({x_dt, "f32"}):
            x = _draw((48, 160), x_dt, rng, 3.0, specials=False)
            g = _draw((48, 160), out_dt, rng, 1.0, specials=False)
            p = rng.uniform(0, 1, 48).astype(np.float32)
            o = orc.router_weight_bwd(g, out_dt, x, x_dt, p)
            tx = _np_to_torch(x, x_dt).float().requires_grad_(True)
            tp = torch.from_numpy(p)[:, None].clone().requires_grad_(True)
            y = (tx * tp).to(DT_TORCH[out_dt])
            y.backward(_np_to_torch(g, out_dt))
            assert _same_bits(o["grad_x"], _torch_to_np(tx.grad, x_dt), x_dt).all(), \
                f"router grad_x {x_dt}/{out_dt}"
            exact = (_np_to_torch(g, out_dt).double() * _np_to_torch(x, x_dt).double()).sum(-1).numpy()
            bad = grad_probs_violations(o["grad_probs"], exact, o["row_scale"])
            assert bad.size == 0, f"router grad_probs {x_dt}/{out_dt}"
            bad = grad_probs_violations(tp.grad.reshape(-1).numpy(), exact, o["row_scale"])
            assert bad.size == 0, "torch's own fp32 sum must meet the same bar"
            assert np.allclose(o["grad_probs_f64"], exact, rtol=0, atol=1e-6 * o["row_scale"].max())
    # without grad_probs nothing reads x
    o = orc.router_weight_bwd(_draw((4, 8), "bf16", rng), "bf16", None, "bf16",
                              np.ones(4, np.float32), want_grad_probs=False)
    assert o["grad_probs"] is None


def pin_squared_relu_no_clamp(orc):
    rng = np.random.default_rng(4)
    x = _draw((96, 256), "bf16", rng, 8.0)
    p = rng.uniform(0, 1, 96).astype(np.float32)
    got = orc.squared_relu_probs(x, p)
    tx = _np_to_torch(x, "bf16")
    sq = torch.relu(tx) * torch.relu(tx)          # a bf16 tensor op: fp32 product, one rounding
    want = _torch_to_np(sq.float() * torch.from_numpy(p)[:, None], "bf16")
    assert _same_bits(got, want, "bf16").all(), "squared relu without clamp"
    # the square really is rounded to bf16 first: a single fp32 chain differs somewhere
    one = _torch_to_np(torch.relu(tx.float()) ** 2 * torch.from_numpy(p)[:, None], "bf16")
    assert not (got == one).all()


def pin_squared_relu_clamp(orc):
    rng = np.random.default_rng(5)
    x = _draw((64, 256), "bf16", rng, 8.0, specials=False)
    p = rng.uniform(0.01, 1, 64).astype(np.float32)
    for s in (0.5, 3.0, 20.0):
        got = orc.squared_relu_probs(x, p, clamp_scale=s)
        xd = torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64))
        want = torch.relu(s * torch.tanh(xd / s)) ** 2 * torch.from_numpy(p.astype(np.float64))[:, None]
        assert_within_ulp(got, _torch_to_np(want.float(), "bf16"), 1, f"soft clamp s={s}")
        assert bf16_bits_to_f32(got).max() <= s * s * 1.0001, "soft clamp bound"
    # a large scale reduces the soft clamp to the identity: relu(x)^2 * p in fp32
    got = orc.squared_relu_probs(x, p, clamp_scale=1e6)
    want = torch.relu(torch.from_numpy(bf16_bits_to_f32(x))) ** 2 * torch.from_numpy(p)[:, None]
    assert_within_ulp(got, _torch_to_np(want, "bf16"), 1, "s -> inf")


def pin_squared_relu_rows(orc):
    rng = np.random.default_rng(6)
    x = _draw((40, 64), "bf16", rng, 3.0, specials=False)
    p = rng.uniform(0, 1, 40).astype(np.float32)
    full = orc.squared_relu_probs(x, p, clamp_scale=2.0)
    perm = rng.permutation(40).astype(np.int32)
    assert np.array_equal(orc.squared_relu_probs(x, p, clamp_scale=2.0, permutation_map=perm),
                          orc.squared_relu_probs(x, p[perm], clamp_scale=2.0))
    for k in (0, 13, 40):
        for zp in (False, True):
            y = orc.squared_relu_probs(x, p, clamp_scale=2.0, n_used=k, zero_padding=zp)
            assert np.array_equal(y[:k], full[:k])
            assert np.all(y[k:] == (0 if zp else 0xFFFF))
    pm = np.arange(40, dtype=np.int32)
    pm[[2, 9]] = [-1, 40]
    y = orc.squared_relu_probs(x, p, clamp_scale=2.0, permutation_map=pm, zero_padding=True)
    assert np.all(y[[2, 9]] == 0) and np.array_equal(np.delete(y, [2, 9], 0), np.delete(full, [2, 9], 0))


def _bf16_values(rng, shape, scale, min_abs):
    """bf16 bit patterns ~ N(0, scale^2) kept at least min_abs away from 0 (the kink)."""
    v = rng.standard_normal(shape) * scale
    v = np.where(np.abs(v) < min_abs, np.copysign(min_abs, v) + v, v).astype(np.float32)
    return _torch_to_np(torch.from_numpy(v), "bf16")


def _sqrelu_fwd64(xd, pd, s, round_square):
    """The page's forward in fp64 (no final rounding). Without the clamp the square of
    the bf16 ReLU output is rounded to bf16 when round_square is set."""
    if s is None:
        sq = np.maximum(xd, 0.0) ** 2
        if round_square:
            sq = bf16_bits_to_f32(_torch_to_np(torch.from_numpy(sq.astype(np.float32)), "bf16")).astype(np.float64)
        return sq * pd
    return np.maximum(s * np.tanh(xd / s), 0.0) ** 2 * pd


def pin_squared_relu_bwd_fd(orc):
    """grad_x = g * dy/dx and grad_probs = sum g * dy/dp by central differences in fp64.
    Past |x / s| = 5 a difference of the saturated forward is rounding noise, so there
    dy/dx comes from the textbook derivative of tanh, 1 / cosh^2, in fp64 (accurate to
    |z| ~ 700). With s = 0.7, |x / s| reaches ~25: sech^2 down to 1e-21, where
    1 - tanh^2 from an fp32 tanh has no digits left."""
    rng = np.random.default_rng(11)
    rows, hidden = 8, 64
    x = _bf16_values(rng, (rows, hidden), 4.0, 1e-2)
    g = _torch_to_np(torch.from_numpy(rng.standard_normal((rows, hidden)).astype(np.float32)), "bf16")
    p = rng.uniform(0.1, 1.0, rows).astype(np.float32)
    xd = bf16_bits_to_f32(x).astype(np.float64)
    gd = bf16_bits_to_f32(g).astype(np.float64)
    pd = p.astype(np.float64)[:, None]
    for s in (None, 0.7, 4.0):
        o = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=s)
        h = 1e-6 * np.maximum(1.0, np.abs(xd))
        dydx = (_sqrelu_fwd64(xd + h, pd, s, False) - _sqrelu_fwd64(xd - h, pd, s, False)) / (2 * h)
        if s is not None:
            z = xd / s
            far = np.abs(z) > 5.0
            assert s > 1.0 or far.sum() > 20, "the small scale must reach deep saturation"
            exact = 2.0 * np.maximum(s * np.tanh(z), 0.0) / np.cosh(z) ** 2 * pd
            dydx = np.where(far, exact, dydx)
        want = _torch_to_np(torch.from_numpy((gd * dydx).astype(np.float32)), "bf16")
        assert_within_ulp(o["grad_x"], want, 1, f"squared relu grad_x by differences, s={s}")
        hp = 1e-6
        lp = (gd * _sqrelu_fwd64(xd, pd + hp, s, True)).sum(1)
        lm = (gd * _sqrelu_fwd64(xd, pd - hp, s, True)).sum(1)
        fd = (lp - lm) / (2 * hp)
        bad = grad_probs_violations(o["grad_probs"], fd, o["row_scale"])
        assert bad.size == 0, f"squared relu grad_probs by differences, s={s}"
        assert np.all(np.abs(o["grad_probs_f64"] - fd) <= 1e-6 * o["row_scale"] + 1e-9)  # fp32 terms


def pin_squared_relu_bwd_structure(orc):
    rng = np.random.default_rng(12)
    rows, hidden = 16, 96
    x = _bf16_values(rng, (rows, hidden), 3.0, 1e-3)
    g = _torch_to_np(torch.from_numpy(rng.standard_normal((rows, hidden)).astype(np.float32)), "bf16")
    p = rng.uniform(0.05, 1.0, rows).astype(np.float32)
    plain = orc.squared_relu_probs_bwd(x, p, g)
    # a huge scale makes the soft clamp the identity: the unclamped gradient
    big = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=1e30)
    assert_within_ulp(big["grad_x"], plain["grad_x"], 1, "s -> inf")
    assert np.array_equal(plain["grad_x"][bf16_bits_to_f32(x) <= 0], np.zeros((bf16_bits_to_f32(x) <= 0).sum(), np.uint16))
    for s in (None, 2.0):
        o = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=s)
        # linear in g: doubling grad_y (exact in bf16) doubles grad_x exactly
        g2 = _torch_to_np(_np_to_torch(g, "bf16").float() * 2, "bf16")
        o2 = orc.squared_relu_probs_bwd(x, p, g2, clamp_scale=s)
        a, b = bf16_bits_to_f32(o["grad_x"]), bf16_bits_to_f32(o2["grad_x"])
        ok = np.abs(a) > 1e-30
        assert np.array_equal(b[ok], 2 * a[ok]), f"linear in g, s={s}"
        # grad_probs does not depend on p; grad_x vanishes with p
        o3 = orc.squared_relu_probs_bwd(x, np.zeros_like(p), g, clamp_scale=s)
        assert np.array_equal(o3["grad_probs"], o["grad_probs"]), f"grad_probs free of p, s={s}"
        assert np.all(bf16_bits_to_f32(o3["grad_x"]) == 0)
    # without the clamp, y_pre is the forward's output at p = 1 (the bf16 square)
    y1 = bf16_bits_to_f32(orc.squared_relu_probs(x, np.ones(rows, np.float32))).astype(np.float64)
    want = (bf16_bits_to_f32(g).astype(np.float32) * y1.astype(np.float32)).astype(np.float64).sum(1)
    assert np.all(np.abs(plain["grad_probs_f64"] - want) <= 1e-12 * plain["row_scale"]), "y_pre is the bf16 square"
    # masks and special values: x <= 0, -0, -inf and NaN give +0; +inf saturates the clamp
    sp = np.array([0x0000, 0x8000, 0xFF80, 0x7FC0, 0xC040, 0x7F80, 0x3F80, 0x0001], np.uint16)
    xs = np.tile(sp, (2, 1))
    gs = np.full_like(xs, 0xBF80)                                  # grad_y = -1
    ps = np.array([0.5, 0.25], np.float32)
    for s in (None, 1.5):
        o = orc.squared_relu_probs_bwd(xs, ps, gs, clamp_scale=s)
        assert np.all(o["grad_x"][:, :5] == 0x0000), f"mask gives +0, s={s}"
        if s is None:
            assert np.all(o["grad_x"][:, 5] == 0xFF80), "(g p) (2 inf) = -inf"
        else:
            assert np.all(o["grad_x"][:, 5] == 0x8000), "sech^2(inf) = 0: -0"
        assert np.all(bf16_bits_to_f32(o["grad_x"][:, 6]) < 0)
        assert np.all(np.isnan(o["grad_probs"])), "the row holds a NaN input"


def pin_squared_relu_bwd_rows(orc):
    rng = np.random.default_rng(13)
    rows, hidden = 40, 64
    x = _bf16_values(rng, (rows, hidden), 3.0, 1e-3)
    g = _torch_to_np(torch.from_numpy(rng.standard_normal((rows, hidden)).astype(np.float32)), "bf16")
    p = rng.uniform(0, 1, rows).astype(np.float32)
    full = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=2.0)
    perm = rng.permutation(rows).astype(np.int32)
    pm = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=2.0, permutation_map=perm)
    ref = orc.squared_relu_probs_bwd(x, p[perm], g, clamp_scale=2.0)
    assert np.array_equal(pm["grad_x"], ref["grad_x"]), "p gathered through the map"
    assert np.array_equal(pm["grad_probs"][perm], ref["grad_probs"]), "grad_probs scattered to the slot"
    for k in (0, 13, rows):
        for zp in (False, True):
            o = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=2.0, n_used=k, zero_padding=zp)
            assert np.array_equal(o["grad_x"][:k], full["grad_x"][:k])
            assert np.all(o["grad_x"][k:] == (0 if zp else 0xFFFF))
            assert np.array_equal(o["grad_probs"][:k], full["grad_probs"][:k])
            assert np.all(o["grad_probs"][k:] == -12345.5), "slots that are not live stay untouched"
    m = np.arange(rows, dtype=np.int32)
    m[[2, 9]] = [-1, rows]
    o = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=2.0, permutation_map=m, zero_padding=True)
    assert np.all(o["grad_x"][[2, 9]] == 0)
    assert np.array_equal(np.delete(o["grad_x"], [2, 9], 0), np.delete(full["grad_x"], [2, 9], 0))
    assert np.all(o["grad_probs"][[2, 9]] == -12345.5)


def pin_unpermute(orc):
    rng = np.random.default_rng(7)
    tokens, E, hidden, erows = 50, 6, 48, 120
    eo = _draw((erows, hidden), "bf16", rng, 2.0, specials=False)
    im = rng.integers(-1, erows, size=(tokens, E)).astype(np.int32)
    im[rng.random((tokens, E)) < 0.4] = -1
    im[0] = -1                       # a token with no local contribution
    im[1, 2] = erows + 5             # out of range: skipped
    for out_dt in ("f32", "bf16"):
        got = orc.unpermute(eo, im, out_dt)
        ef = bf16_bits_to_f32(eo)
        acc = np.zeros((tokens, hidden), np.float32)
        for e in range(E):           # running fp32 sums in increasing expert id
            rows = im[:, e]
            ok = (rows >= 0) & (rows < erows)
            acc[ok] = acc[ok] + ef[rows[ok]]
        want = acc if out_dt == "f32" else _torch_to_np(torch.from_numpy(acc), "bf16")
        assert _same_bits(got, want, out_dt).all(), f"unpermute {out_dt}"
    # one contribution per token copies the row exactly
    im1 = np.full((tokens, E), -1, np.int32)
    im1[np.arange(tokens), rng.integers(0, E, tokens)] = rng.integers(0, erows, tokens)
    got = orc.unpermute(eo, im1, "bf16")
    assert np.array_equal(got, eo[im1.max(axis=1)])
    # tokens at or past valid_tokens are untouched
    got = orc.unpermute(eo, im, "bf16", valid_tokens=17)
    assert np.all(got[17:] == 0xFFFF) and np.array_equal(got[:17], orc.unpermute(eo, im, "bf16")[:17])
    assert np.all(orc.unpermute(eo, im, "bf16", valid_tokens=-3) == 0xFFFF)
    # the order is increasing expert id: contributions 2^24, 1, -2^24 sum to 0 in that
    # order (2^24 + 1 rounds to 2^24 in fp32) and to 1 in the reverse order
    big = np.zeros((3, hidden), np.uint16)
    big[0] = 0x4B80                  # 2^24
    big[1] = 0x3F80                  # 1
    big[2] = 0xCB80                  # -2^24
    order = orc.unpermute(big, np.array([[0, 1, 2], [2, 1, 0]], np.int32), "f32")
    assert np.all(order[0] == 0.0) and np.all(order[1] == 1.0), "expert order of the fp32 sum"
    # order matters only through rounding: reversing the experts stays within fp32 error
    rev = orc.unpermute(eo, im[:, ::-1].copy(), "f32")
    fwd = orc.unpermute(eo, im, "f32")
    assert np.allclose(rev, fwd, rtol=0, atol=E * 2 * math.ldexp(1, -24) * np.abs(fwd).max() + 1e-30)


def pin_thread_count_invariance(orc):
    """Rows run in static blocks over threads; the arithmetic of a row does not depend on
    which thread runs it, so every output bit is the same for 1, 3 and 7 threads (with
    more row blocks than rows for the small cases, and a residual add large enough to
    span several element blocks)."""
    rng = np.random.default_rng(11)
    rows, hidden = 203, 40
    x = _draw((rows, hidden), "bf16", rng, 3.0)
    g = _draw((rows, hidden), "bf16", rng, 1.0)
    p = rng.random(rows).astype(np.float32)
    m = rng.permutation(rows).astype(np.int32)
    m[[4, 50]] = [-1, rows + 2]
    n = 3 * 65536 + 17
    e, sh, r = (_draw((n,), "bf16", rng, 1.0) for _ in range(3))
    eo = _draw((300, hidden), "bf16", rng, 2.0, specials=False)
    im = rng.integers(-1, 300, size=(rows, 8)).astype(np.int32)

    def run(t):
        outs = [orc.residual_add(e, sh, r, "bf16", threads=t),
                orc.router_weight_fwd(x, "bf16", p, "f32", threads=t)]
        rb = orc.router_weight_bwd(g, "bf16", x, "bf16", p, threads=t)
        outs += [rb["grad_x"], rb["grad_probs"], rb["grad_probs_f64"], rb["row_scale"]]
        for s in (None, 4.0):
            outs.append(orc.squared_relu_probs(x, p, clamp_scale=s, n_used=190, permutation_map=m,
                                               zero_padding=s is None, threads=t))
            sb = orc.squared_relu_probs_bwd(x, p, g, clamp_scale=s, n_used=190, permutation_map=m,
                                            zero_padding=s is not None, threads=t)
            outs += [sb["grad_x"], sb["grad_probs"], sb["grad_probs_f64"], sb["row_scale"]]
        outs += [orc.unpermute(eo, im, "f32", threads=t), orc.unpermute(eo, im, "bf16", valid_tokens=150, threads=t)]
        return outs

    ref = run(1)
    for t in (3, 7):
        for i, (a, b) in enumerate(zip(ref, run(t))):
            assert a.tobytes() == b.tobytes(), f"output {i} changed with {t} threads"


ALL_PINS = [pin_f16_conversions, pin_residual_add, pin_router_weight_fwd, pin_router_weight_bwd,
            pin_squared_relu_no_clamp, pin_squared_relu_clamp, pin_squared_relu_rows,
            pin_squared_relu_bwd_fd, pin_squared_relu_bwd_structure, pin_squared_relu_bwd_rows,
            pin_unpermute, pin_thread_count_invariance]
