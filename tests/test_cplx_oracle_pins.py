"""The fp64 complex-A forward oracle checked against the real oracle, closed
forms and invariants."""

import pytest

import cplx_oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_CPLX_PINS, ids=lambda f: f.__name__)
def test_cplx_pin(oracle_lib, pin):
    pin(oracle_lib)
