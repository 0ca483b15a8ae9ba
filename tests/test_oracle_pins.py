"""Every oracle pin (tests/oracle_pins.py) run against the oracle built from oracle/xr_oracle.c."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_pin_list_is_complete():
    assert len(oracle_pins.ALL_PINS) >= 18
