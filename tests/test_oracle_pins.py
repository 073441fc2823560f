"""The CPU oracle against facts fixed by the mathematics (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
