"""Prefill-to-decode hand-off and the state update, against the oracle.

The 32k-token workload: scan the first 32768 steps with final-state export,
then advance 64 decode steps on fresh inputs with the state update, and
compare every decode output and the final state with one oracle run over all
32832 steps (sampled channels).
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, sample_channels, to_np
from mamba_selective_scan_amd.inputs import WORKLOADS, generate, generate_workload, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _decode_steps(mss, dx, state, t_from, t_to):
    outs = []
    for t in range(t_from, t_to):
        y = mss.selective_state_update(state, dx["u"][:, :, t], dx["delta_raw"][:, :, t],
                                       dx["A_log"], dx["B"][:, :, t], dx["C"][:, :, t],
                                       D=dx["D"], z=dx["z"][:, :, t], dt_bias=dx["dt_bias"])
        outs.append(y)
    return outs


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_long_handoff(mss, io):
    import torch
    w = WORKLOADS["long_handoff"]
    L, extra = w.seqlen, w.decode_steps
    note(f"long_handoff {io}: generating L+{extra}")
    x = generate_workload(w, seed=0)
    dx = to_torch(x, device(), io)
    pre = {k: (v[:, :, :L] if k in ("u", "delta_raw", "z", "B", "C") else v) for k, v in dx.items()}
    note("long_handoff: scan prefill")
    out, state = mss.selective_scan_fwd(pre["u"], pre["delta_raw"], pre["A_log"], pre["B"],
                                        pre["C"], D=pre["D"], z=pre["z"], dt_bias=pre["dt_bias"],
                                        return_final_state=True)
    note("long_handoff: 64 decode steps")
    outs = _decode_steps(mss, dx, state, L, L + extra)
    torch.cuda.synchronize()
    chans = sample_channels(w.batch, w.dim, 64)
    note(f"long_handoff: oracle over L+{extra} on {len(chans)} channels")
    ref_out, ref_fin = oracle.scan_channels(dx, chans)
    tol = 1e-4 if io == "f32" else 2e-2
    got_pre = np.stack([to_np(out[b, d]) for b, d in chans])
    check(f"handoff {io} prefill out", got_pre, ref_out[:, :L], tol)
    got_dec = np.stack([[float(o[b, d]) for o in outs] for b, d in chans])
    check(f"handoff {io} decode out", got_dec, ref_out[:, L:], tol)
    got_fin = np.stack([to_np(state[b, d]) for b, d in chans])
    check(f"handoff {io} final state", got_fin, ref_fin, tol)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dstate", [16, 5])
@pytest.mark.parametrize("shape", [(3, 200), (1, 7), (8, 5120)])
def test_state_update_matches_oracle(mss, io, dstate, shape):
    import torch
    batch, dim = shape
    note(f"state_update {io} N={dstate} B={batch} D={dim}")
    x = generate(batch, dim, 1, dstate, seed=11)
    dx = to_torch(x, device(), io)
    g = torch.Generator().manual_seed(3)
    state = torch.randn(batch, dim, dstate, generator=g).to(device())
    s0 = state.clone()
    y = mss.selective_state_update(state, dx["u"][:, :, 0], dx["delta_raw"][:, :, 0], dx["A_log"],
                                   dx["B"][:, :, 0], dx["C"][:, :, 0], D=dx["D"],
                                   z=dx["z"][:, :, 0], dt_bias=dx["dt_bias"])
    torch.cuda.synchronize()
    ref_y, ref_s = oracle.state_update(s0, dx["u"][:, :, 0], dx["delta_raw"][:, :, 0], dx["A_log"],
                                       dx["B"][:, :, 0], dx["C"][:, :, 0], D=dx["D"],
                                       z=dx["z"][:, :, 0], dt_bias=dx["dt_bias"])
    tol = 1e-4 if io == "f32" else 2e-2
    check("step out", to_np(y), ref_y, tol)
    check("step state", to_np(state), ref_s, 1e-4)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("big_bias", [False, True])
def test_state_update_softplus_upper_range(mss, io, big_bias):
    """The decode step with delta_raw + dt_bias over [-40, 40] (a dense grid
    through 19.5..20.5, values above 30; dt_bias 0 or 25): 342 steps, each on
    every channel, against the oracle step by step."""
    import torch
    from mamba_selective_scan_amd.inputs import softplus_range_delta
    batch, dim, N, steps = 3, 200, 16, 342
    note(f"state_update softplus upper range {io} big_bias={big_bias}")
    x = generate(batch, dim, steps, N, seed=13)
    x["delta_raw"], x["dt_bias"] = softplus_range_delta(batch, dim, steps, seed=13,
                                                        big_bias=big_bias)
    dx = to_torch(x, device(), io)
    g = torch.Generator().manual_seed(5)
    state = torch.randn(batch, dim, N, generator=g).to(device())
    ref_state = to_np(state)
    outs = _decode_steps(mss, dx, state, 0, steps)
    torch.cuda.synchronize()
    ref_outs = []
    for t in range(steps):
        y, ref_state = oracle.state_update(ref_state, dx["u"][:, :, t], dx["delta_raw"][:, :, t],
                                           dx["A_log"], dx["B"][:, :, t], dx["C"][:, :, t],
                                           D=dx["D"], z=dx["z"][:, :, t], dt_bias=dx["dt_bias"])
        ref_outs.append(y)
    tol = 1e-4 if io == "f32" else 2e-2
    check(f"step softplus range {io} out", to_np(torch.stack(outs, dim=2)),
          np.stack(ref_outs, axis=2), tol)
    check(f"step softplus range {io} state", to_np(state), ref_state, tol)


def test_step_sequence_equals_scan(mss):
    """Iterating the state update over a sequence reproduces the scan."""
    import torch
    note("step sequence == scan")
    x = generate(2, 70, 40, 16, seed=4)
    dx = to_torch(x, device(), "f32")
    out, fin = mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                      D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                      return_final_state=True)
    state = torch.zeros(2, 70, 16, device=device())
    outs = _decode_steps(mss, dx, state, 0, 40)
    torch.cuda.synchronize()
    check("steps vs scan out", to_np(torch.stack(outs, dim=2)), to_np(out), 1e-5)
    check("steps vs scan state", to_np(state), to_np(fin), 1e-5)
