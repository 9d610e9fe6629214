"""The fp64 conv1d oracle checked against library filters, closed forms and
invariants."""

import pytest

import conv_oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_CONV_PINS, ids=lambda f: f.__name__)
def test_conv_pin(oracle_lib, pin):
    pin(oracle_lib)
