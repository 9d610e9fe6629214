"""The fp64 oracle checked against closed forms, brute force and invariants."""

import pytest

import oracle_pins as P


def test_scalars(oracle_lib):
    P.pin_scalars(oracle_lib)


def test_brute_force_unrolled_mpmath(oracle_lib):
    P.pin_brute_force(oracle_lib)


def test_geometric_closed_form(oracle_lib):
    P.pin_geometric(oracle_lib)


def test_chunk_composition(oracle_lib):
    P.pin_chunk_composition(oracle_lib)


def test_step_equals_scan(oracle_lib):
    P.pin_step_equals_scan(oracle_lib)


def test_special_cases(oracle_lib):
    P.pin_special_cases(oracle_lib)


def test_invariants(oracle_lib):
    P.pin_invariants(oracle_lib)


def test_operator_associativity():
    P.pin_operator_associativity()


@pytest.mark.parametrize("threads", [1, 3])
def test_thread_count_does_not_change_result(oracle_lib, threads):
    import numpy as np
    import oracle
    rng = np.random.default_rng(7)
    p = P.rand_problem(rng, 2, 5, 33, 4)
    a, fa = oracle.scan_fwd(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["z"],
                            p["dt_bias"], threads=threads)
    b, fb = oracle.scan_fwd(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["z"],
                            p["dt_bias"], threads=0)
    assert np.array_equal(a, b) and np.array_equal(fa, fb)
