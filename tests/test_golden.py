"""The oracle reproduces the hand-derived worked examples in tests/golden/."""

import numpy as np
import pytest

import golden_cases
import oracle


@pytest.mark.parametrize("name", golden_cases.ALL)
def test_oracle_matches_golden(name, oracle_lib):
    c = golden_cases.load(name)
    if c["kind"] == "conv":
        out, fin = oracle.conv1d_fwd(c["x"], c["w"], c["bias"], silu=False)
    elif c["kind"] == "conv_step":
        out, fin = oracle.conv1d_update(c["state"], c["x"], c["w"], c["bias"], silu=False)
    elif c["kind"] == "scan":
        out, fin = oracle.scan_fwd(c["u"], c["delta_raw"], c["A_log"], c["B"], c["C"], D=c["D"],
                                   delta_softplus=False)
    else:
        out, fin = oracle.state_update(c["state"], c["u"], c["delta_raw"], c["A_log"], c["B"],
                                       c["C"], D=c["D"], delta_softplus=False)
    np.testing.assert_allclose(out, c["y"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(fin, c["final"], rtol=1e-14, atol=1e-14)
