"""The CPU oracle against its pins (closed forms, brute force, library routines, invariants)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
