"""The fp64 backward oracle checked against finite differences, automatic
differentiation, Euler identities and a chained split."""

import pytest

import bwd_oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(oracle_lib, pin):
    pin(oracle_lib)
