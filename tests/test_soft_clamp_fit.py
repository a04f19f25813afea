"""Host checks of the squared-ReLU soft clamp's rational tanh.

The kernel writes relu(s * tanh(x / s)) as x * P(u) / Q(u), clamped to [0, s]; its
coefficients are constants in moe_elementwise.hip. These tests read them from the
source, re-run the fit that produced them, and evaluate the kernel's fp32 operation
order in numpy against float64 tanh: the bound has to hold on the CPU before the GPU
parity tests compare the kernel with the oracle.
"""
import importlib.util
import os
import re

import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "memory_bound_elementwise_amd", "csrc")


def _fit_module():
    spec = importlib.util.spec_from_file_location("fit_tanh_rational",
                                                  os.path.join(CSRC, "fit_tanh_rational.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _kernel_constants():
    src = open(os.path.join(CSRC, "moe_elementwise.hip")).read()
    vals = dict((k, np.float32(float(v))) for k, v in
                re.findall(r"(kTanh[PQ]\d|kTanhUMax) = ([-+0-9.eE]+)f", src))
    p = [vals[f"kTanhP{i}"] for i in range(3)]
    q = [np.float32(1.0)] + [vals[f"kTanhQ{i}"] for i in range(1, 3)]
    return p, q, vals["kTanhUMax"]


def test_constants_come_from_the_fit():
    fit = _fit_module()
    p, q, umax = _kernel_constants()
    pf, qf, err = fit.fit(fit.ZMAX)
    assert err < 7e-5 and 1 - np.tanh(fit.ZMAX) < 7e-5
    assert umax == np.float32(fit.ZMAX * fit.ZMAX)
    assert np.array_equal(np.asarray(p, np.float32), pf.astype(np.float32))
    assert np.array_equal(np.asarray(q, np.float32), qf.astype(np.float32))


def test_fp32_evaluation_within_bound():
    """Under 2^-11 relative on c (6.5e-5 measured), so under 2^-10 on c^2: a result c^2 p
    that far from the exact one rounds to a bf16 neighbour of the exact one's rounding (a
    bf16 ulp is at least 2^-8 of the value), so it is within one ulp of the oracle."""
    fit = _fit_module()
    p, q, umax = _kernel_constants()
    err = fit.worst_relative_error(p, q, umax)
    assert err < 2.0 ** -11 and err < 7e-5


@pytest.mark.parametrize("s", [4.0, 0.5, 1e4])
def test_special_values(s):
    fit = _fit_module()
    p, q, umax = _kernel_constants()
    x = np.array([np.inf, -np.inf, np.nan, -0.0, 0.0, -1e-40, 1e-40, 3e38, -3e38], np.float32)
    got = fit.soft_clamp_relu_fp32(x, s, p, q, umax)
    s32 = np.float32(s)
    assert got[0] == s32 and got[1] == 0.0
    assert np.isnan(got[2])
    assert got[3] == 0.0 and not np.signbit(got[3]) and got[4] == 0.0
    assert got[5] == 0.0 and 0.0 < got[6] <= np.float32(1e-40) * 1.0001
    assert got[7] == s32 and got[8] == 0.0


def test_nearly_monotone_and_saturating():
    """tanh is increasing. The minimax fit equioscillates, so the approximation may step
    down, but by no more than twice its error bound, also where u is held at 5.2^2;
    and it reaches s."""
    fit = _fit_module()
    p, q, umax = _kernel_constants()
    x = np.linspace(0.0, 40.0, 400_001).astype(np.float32)
    got = fit.soft_clamp_relu_fp32(x, 4.0, p, q, umax).astype(np.float64)
    assert np.diff(got).min() >= -1.4e-4 * 4.0
    assert got[-1] == 4.0 and np.all(got[x >= 4.0 * 5.3] == 4.0)
