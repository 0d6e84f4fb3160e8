"""The running float sum oracle (O4) against facts other than itself (CPU only)."""

import pytest

import float_sum_pins
import oracle


@pytest.mark.parametrize("pin", float_sum_pins.ALL_PINS, ids=[p.__name__ for p in float_sum_pins.ALL_PINS])
def test_float_sum_oracle_pin(pin):
    assert pin(oracle.running_float_sums) == []
