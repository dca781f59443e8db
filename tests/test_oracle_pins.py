"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""

import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
