"""Exhaustive per-element sweeps: every bf16 bit pattern of gate (and of up) against
fixed partners, through the HIP path and the oracle. Covers subnormals, +-inf,
NaN, the clamp edges and the far tails of silu."""
import numpy as np
import pytest

from parity import check_parity

pytestmark = pytest.mark.gpu

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)


def _bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)


def _inp(gate_bits, up_bits, p, gy_bits, limit):
    rows, inter = gate_bits.shape
    return {"x": np.ascontiguousarray(np.concatenate([gate_bits, up_bits], axis=1)),
            "probs": np.full(rows, p, dtype=np.float32),
            "grad_y": np.ascontiguousarray(gy_bits),
            "limit": limit, "n_used": None, "permutation_map": None, "zero_padding": False}


@pytest.mark.parametrize("limit", [7.0, float("inf"), 0.5])
@pytest.mark.parametrize("up", [1.0, -7.0, 7.03125, 0.0, -3.25])
@pytest.mark.parametrize("p", [1.0, 0.3])
def test_every_gate_pattern(limit, up, p):
    up_bits = np.full_like(ALL, _bits(up))
    gy = np.full_like(ALL, _bits(1.0))
    check_parity(_inp(ALL, up_bits, p, gy, limit), label=f"gate sweep L={limit} up={up} p={p}")


@pytest.mark.parametrize("limit", [7.0, float("inf")])
@pytest.mark.parametrize("gate", [1.0, -1.28125, 7.0, 7.03125, -50.0, 0.0])
def test_every_up_pattern(limit, gate):
    gate_bits = np.full_like(ALL, _bits(gate))
    gy = np.full_like(ALL, _bits(-0.75))
    check_parity(_inp(gate_bits, ALL, 0.6, gy, limit), label=f"up sweep L={limit} gate={gate}")


@pytest.mark.parametrize("seed", [0, 1])
def test_random_bit_patterns(seed):
    """Gate, up and grad_y drawn as uniform random 16-bit patterns (any class)."""
    rng = np.random.default_rng(seed)
    g = rng.integers(0, 65536, size=(1024, 512), dtype=np.uint32).astype(np.uint16)
    u = rng.integers(0, 65536, size=(1024, 512), dtype=np.uint32).astype(np.uint16)
    gy = rng.integers(0, 65536, size=(1024, 512), dtype=np.uint32).astype(np.uint16)
    inp = _inp(g, u, 0.5, gy, 7.0)
    inp["probs"] = rng.uniform(0, 1, size=1024).astype(np.float32)
    check_parity(inp, label=f"random bits seed={seed}")
