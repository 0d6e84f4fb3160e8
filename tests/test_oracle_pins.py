"""The oracle against facts other than itself (CPU only)."""

import pytest

import oracle_pins


@pytest.fixture(scope="module")
def real():
    return oracle_pins.RealOracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=[p.__name__ for p in oracle_pins.ALL_PINS])
def test_oracle_pin(pin, real):
    assert pin(real) == []
