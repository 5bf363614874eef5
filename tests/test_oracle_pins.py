"""The oracle against its pins (closed forms, brute force, codecs, invariants)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
