"""The seeded input generator: determinism, shapes, layouts and value ranges."""

import numpy as np

from mamba_selective_scan_amd.inputs import WORKLOADS, algorithmic_bytes, generate


def test_deterministic_and_seeded():
    a = generate(2, 8, 33, 4, seed=0)
    b = generate(2, 8, 33, 4, seed=0)
    c = generate(2, 8, 33, 4, seed=1)
    for k in ("u", "delta_raw", "z", "B", "C", "A_log", "D", "dt_bias"):
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["u"], c["u"])


def test_shapes_and_layouts():
    a = generate(2, 8, 33, 4, layout="bdl")
    assert a["u"].shape == (2, 8, 33) and a["B"].shape == (2, 4, 33)
    assert a["u"].flags["C_CONTIGUOUS"]
    b = generate(2, 8, 33, 4, layout="bld")
    assert b["u"].shape == (2, 8, 33) and b["B"].shape == (2, 4, 33)
    assert b["u"].strides[1] == 4 and b["u"].strides[2] == 8 * 4      # d is the unit-stride axis
    assert b["B"].strides[1] == 4 and b["B"].strides[2] == 4 * 4


def test_value_ranges():
    a = generate(1, 4096, 64, 16, seed=3)
    dt = np.log1p(np.exp(a["dt_bias"].astype(np.float64)))
    assert dt.min() >= 1e-3 * 0.999 and dt.max() <= 0.1 * 1.001
    assert np.array_equal(a["A_log"][5], np.log(np.arange(1, 17)).astype(np.float32))
    assert np.all(a["D"] == 1.0)
    assert abs(float(a["delta_raw"].std()) - 0.1) < 0.005
    assert abs(float(a["u"].std()) - 1.0) < 0.02


def test_workload_table():
    w = WORKLOADS["mamba2p8b_layer"]
    assert (w.batch, w.dim, w.seqlen, w.dstate) == (8, 5120, 4096, 16)
    assert algorithmic_bytes(8, 5120, 4096, 16, 4) == 2688917504
    assert WORKLOADS["audio_channel_last"].layout == "bld"
    assert WORKLOADS["long_handoff"].decode_steps == 64
