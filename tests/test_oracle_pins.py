"""The CPU oracle against values fixed independently of it (no GPU needed).

The pins themselves live in ``oracle_pins.py``; its docstring maps each part of
the oracle to the pin that checks it.
"""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
