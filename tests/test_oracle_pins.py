"""The float64 oracle against checks that come from outside it: closed forms,
brute force over explicit sequences, torch's attention, invariances and a
hand-written fixture (the pins live in pins.py)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
