"""bench.py's host-side contract, on the CPU: it refuses more than one GPU,
its kernel-source hashes are stable, and a committed HBM-traffic record is
used only while it matches the kernel sources it was measured on."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_several_gpus(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_source_hash_is_stable():
    for op in bench.KERNEL_SOURCES:
        h = bench.kernel_source_hash(op)
        assert len(h) == 16 and h == bench.kernel_source_hash(op)
    assert bench.kernel_source_hash("scan") != bench.kernel_source_hash("scan_bwd")


def test_traffic_record_requires_matching_sources():
    path = os.path.join(ROOT, "profiles", "traffic_scan_mamba2p8b_layer_f32.json")
    with open(path) as f:
        rec = json.load(f)
    assert rec["algorithmic_bytes_per_launch"] > 0
    assert bench.load_traffic("mamba2p8b_layer", "f32", rec["kernel_source_hash"]) == \
        rec["traffic_bytes_per_launch"]
    assert bench.load_traffic("mamba2p8b_layer", "f32", "0" * 16) is None
    assert bench.load_traffic("no_such_workload", "f32", rec["kernel_source_hash"]) is None


def test_step_bytes():
    # state read + write, four activations, B and C, the parameters
    assert bench.step_bytes(1, 2, 3, 4) == 2 * 1 * 2 * 3 * 4 + 4 * 1 * 2 * 4 + 2 * 1 * 3 * 4 + \
        2 * 3 * 4 + 2 * 2 * 4


def test_valu_instructions_per_element():
    # 5 per state-step (exp2, two multiplies, two FMAs) and 19 per element
    assert bench.valu_instr_per_element(16) == 99
    assert bench.valu_instr_per_element(16, softplus=False, has_z=False) == 84
    assert bench.bwd_valu_instr_per_element(16) == 223
    assert bench.complex_valu_instr_per_element(16) == 259


def test_cold_cache_sets():
    from mamba_selective_scan_amd.inputs import WORKLOADS, algorithmic_bytes
    llc = bench.LLC_BYTES
    for name, w in WORKLOADS.items():
        nbytes = algorithmic_bytes(w.batch, w.dim, w.seqlen, w.dstate, 4, final_state=True)
        n = bench.cache_sets(nbytes)
        if nbytes >= 3 * llc:
            assert n == 1, name
        else:
            assert 8 <= n <= 256, name
    # the 130m-layer shape (50.7 MB) rotates 16 sets, over 3x the cache
    w = WORKLOADS["mamba130m_layer"]
    nbytes = algorithmic_bytes(w.batch, w.dim, w.seqlen, w.dstate, 4, final_state=True)
    assert bench.cache_sets(nbytes) == 16 and 16 * nbytes >= 3 * llc


def test_host_cpu_model():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
