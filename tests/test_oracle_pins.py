"""CPU checks that pin the oracle to the definitions (no GPU needed)."""

import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
