"""Comparison helpers for bf16 bit patterns and fp32 row sums (test infrastructure).

``ulp_distance`` is the distance between two bf16 values counted in representable
steps: bit patterns are mapped to a monotone integer line on which +0 and -0 are
the same point, so "within 1 bf16 ulp" means a distance of at most 1. NaN matches
only NaN.
"""
from __future__ import annotations

import numpy as np


def _ordinal(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Elementwise distance in bf16 steps; 0 where both are NaN, huge where only one is."""
    a_bits = np.asarray(a_bits, dtype=np.uint16)
    b_bits = np.asarray(b_bits, dtype=np.uint16)
    d = np.abs(_ordinal(a_bits) - _ordinal(b_bits))
    na, nb = is_nan(a_bits), is_nan(b_bits)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 20, d)
    return d


def assert_within_ulp(got: np.ndarray, want: np.ndarray, max_ulp: int = 1, what: str = "") -> None:
    d = ulp_distance(got, want)
    bad = np.argwhere(d > max_ulp)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {bad.shape[0]} of {d.size} elements differ by more than {max_ulp} bf16 ulp; "
            f"first at {i}: got 0x{int(got[i]):04x} want 0x{int(want[i]):04x} (max {int(d.max())})")


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def grad_probs_violations(got: np.ndarray, want_f64: np.ndarray, row_scale: np.ndarray,
                          rtol: float = 1e-5, atol: float = 1e-6) -> np.ndarray:
    """Indices where |got - want| > atol + rtol * S (S = the row's sum of |terms|).

    The relative part is taken against the row's condition scale S rather than
    |want|: on rows where the terms cancel, fp32 rounding of the terms alone can
    move the sum by more than 1e-5 of its (small) value whatever the summation
    order, while the error stays a tiny fraction of S.
    """
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want_f64)
    tol = atol + rtol * row_scale
    return np.flatnonzero(~(err <= tol))
