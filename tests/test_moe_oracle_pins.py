"""The MoE-ops oracle against values fixed independently of it (no GPU needed)."""
import pytest

import oracle.moe as moe
from moe_oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return moe.get()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
