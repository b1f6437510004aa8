"""The CPU oracle against its pins (closed forms, brute force, library routines, worked examples)."""
import pytest

import oracle
from pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
