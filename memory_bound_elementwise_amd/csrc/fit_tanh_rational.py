"""Fit the rational soft-clamp approximation used by the squared-ReLU kernel.

tanh(z) / z is approximated by P(u) / Q(u), u = z^2, P and Q of degree 2 with
Q(0) = 1, minimax in relative error over 0 <= z <= ZMAX. ZMAX = 5.2 balances the fit's
error (6.5e-5) against the saturation error 1 - tanh(ZMAX) (6.1e-5): the kernel holds u
at ZMAX^2 and clamps the result to s beyond it. The fit is Loeb's
linearisation (solve P - f Q = 0 in least squares, weighted by 1 / Q of the last
pass) with Lawson reweighting (weights grow with the local error) to approach the
equioscillating minimax solution. It prints the coefficients rounded to fp32 as
they appear in moe_elementwise.hip, and the worst relative error of the kernel's
fp32 evaluation order against float64 tanh.

    python3 fit_tanh_rational.py [zmax]
"""
import sys

import numpy as np

ZMAX = 5.2
DEG_P = DEG_Q = 2


def fit(zmax: float, deg_p: int = DEG_P, deg_q: int = DEG_Q, iters: int = 200):
    z = np.unique(np.concatenate([np.linspace(0.0, zmax, 20000),
                                  zmax * (1.0 - np.geomspace(1e-9, 1.0, 2000))]))
    u = z * z
    f = np.ones_like(z)
    f[z > 0] = np.tanh(z[z > 0]) / z[z > 0]
    w = np.ones_like(u)
    q = np.zeros(deg_q + 1)
    q[0] = 1.0
    for _ in range(iters):
        q_prev = np.polyval(q[::-1], u)
        a = np.hstack([u[:, None] ** np.arange(deg_p + 1),
                       -f[:, None] * u[:, None] ** np.arange(1, deg_q + 1)])
        scale = w / (np.abs(q_prev) * f)
        sol, *_ = np.linalg.lstsq(a * scale[:, None], f * scale, rcond=None)
        p = sol[:deg_p + 1]
        q = np.concatenate([[1.0], sol[deg_p + 1:]])
        err = np.polyval(p[::-1], u) / np.polyval(q[::-1], u) / f - 1.0
        w = w * np.sqrt(np.abs(err))
        w /= w.max()
    return p, q, float(np.abs(err).max())


def _fma(a, b, c):
    # a * b is exact in float64 for fp32 operands; one rounding of the sum, then to fp32
    return (np.asarray(a, np.float64) * b + c).astype(np.float32)


def soft_clamp_relu_fp32(x, s, p, q, umax):
    """The kernel's order of fp32 operations (the reciprocal taken as correctly rounded)."""
    f32 = np.float32
    x = np.asarray(x, f32)
    s = f32(s)
    inv_s = f32(1.0) / s
    with np.errstate(over="ignore", invalid="ignore"):   # +-inf inputs and overflow are part of the check
        z = (x * inv_s).astype(f32)
        u = np.fmin((z * z).astype(f32), f32(umax))
        pn = np.full_like(u, p[-1])
        for c in p[-2::-1]:   # Horner, one fma per coefficient, as the kernel
            pn = _fma(pn, u, c)
        qd = np.full_like(u, q[-1])
        for c in q[-2::-1]:
            qd = _fma(qd, u, c)
        c = (x * (pn * (f32(1.0) / qd)).astype(f32)).astype(f32)
        # maximum / minimum propagate NaN
        return np.maximum(np.minimum(c, s), f32(0.0))


def worst_relative_error(p, q, umax, scales=(4.0, 1.0, 0.37, 1000.0, 3e-5)):
    worst = 0.0
    for s in scales:
        s32 = float(np.float32(s))
        x = np.concatenate([np.linspace(-30 * s32, 30 * s32, 1_000_001),
                            np.geomspace(1e-38, 60 * s32, 500_000)]).astype(np.float32)
        got = soft_clamp_relu_fp32(x, s32, p, q, umax).astype(np.float64)
        want = np.maximum(s32 * np.tanh(x.astype(np.float64) / s32), 0.0)
        pos = want > 0
        if np.any((got > 0) != pos):
            raise AssertionError(f"sign mismatch at scale {s}")
        worst = max(worst, float(np.max(np.abs(got[pos] - want[pos]) / want[pos])))
    return worst


def main():
    zmax = float(sys.argv[1]) if len(sys.argv) > 1 else ZMAX
    p, q, err = fit(zmax)
    p32, q32 = p.astype(np.float32), q.astype(np.float32)
    umax = np.float32(zmax * zmax)
    print(f"minimax relative error of P/Q: {err:.3g}; 1 - tanh(zmax): {1 - np.tanh(zmax):.3g}")
    for i, c in enumerate(p32):
        print(f"kTanhP{i} = {float(c)!r}f")
    for i, c in enumerate(q32[1:], 1):
        print(f"kTanhQ{i} = {float(c)!r}f")
    print(f"kTanhUMax = {float(umax)!r}f")
    print(f"fp32 evaluation, worst relative error of the clamp: {worst_relative_error(p32, q32, umax):.3g}")


if __name__ == "__main__":
    main()
