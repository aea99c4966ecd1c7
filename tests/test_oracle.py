"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    oracle.compile_oracle()
    return oracle.Oracle(oracle.LIB_PATH)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
