"""Chunk states: the forward's record of the state entering every 16-step chunk
of logical time, and the backward that reads them instead of recomputing them.

The oracle's value for chunk q is the final state of the fp64 forward run on
the first 16 q logical steps (the initial state for q = 0); in reverse time the
logical steps are the storage steps from the end.  Slots n >= dstate hold 0.
Tolerances as for the final state (test_parity.py): 1e-4 for fp32 I/O, 2e-2
for bf16.  The backward given the recorded states is checked against the
backward oracle and against the same backward run without them.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import generate, to_torch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _np(a):
    return None if a is None else to_np(a)


def _oracle_chunk_states(dx, h0, reverse):
    """States entering each 16-step chunk, from oracle runs on prefixes."""
    flip = (lambda a: None if a is None else np.ascontiguousarray(a[:, :, ::-1])) if reverse \
        else (lambda a: a)
    x = {k: flip(_np(dx[k])) for k in ("u", "delta_raw", "B", "C", "z")}
    bsz, dim, seqlen = x["u"].shape
    dstate = dx["A_log"].shape[1]
    nq = (seqlen + 15) // 16
    ref = np.zeros((nq, bsz, dim, 16))
    ref[0, :, :, :dstate] = 0.0 if h0 is None else _np(h0)
    for q in range(1, nq):
        t = 16 * q
        _, fin = oracle.scan_fwd(x["u"][:, :, :t], x["delta_raw"][:, :, :t], _np(dx["A_log"]),
                                 x["B"][:, :, :t], x["C"][:, :, :t], D=_np(dx["D"]),
                                 z=None if x["z"] is None else x["z"][:, :, :t],
                                 dt_bias=_np(dx["dt_bias"]), h0=_np(h0))
        ref[q, :, :, :dstate] = fin
    return ref


def _case(mss, name, batch, dim, seqlen, dstate=16, layout="bdl", io="f32", reverse=False,
          h0=False, a_log="ladder", seed=3):
    import torch
    note(f"chunk states {name}: B={batch} D={dim} L={seqlen} N={dstate} {layout} {io} "
         f"reverse={reverse} h0={h0}")
    x = generate(batch, dim, seqlen, dstate, layout, seed=seed, a_log=a_log)
    dx = to_torch(x, device(), io)
    init = (torch.randn(batch, dim, dstate, generator=torch.Generator().manual_seed(seed + 1))
            .to(device()) if h0 else None)
    out, fin, states = mss.selective_scan_fwd(
        dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], D=dx["D"], z=dx["z"],
        dt_bias=dx["dt_bias"], initial_state=init, return_final_state=True,
        return_chunk_states=True, reverse=reverse)
    torch.cuda.synchronize()
    assert tuple(states.shape) == mss.chunk_states_shape(dx["u"])
    ref = _oracle_chunk_states(dx, init, reverse)
    check(f"chunk states {name}", to_np(states), ref, TOL[io])
    assert np.all(to_np(states)[:, :, :, dstate:] == 0.0)
    return dx, init, states


@pytest.mark.parametrize("seqlen", [1, 16, 17, 50, 100])
def test_chunk_states_bdl(mss, seqlen):
    # L = 50: the element-wise tail pass starts at step 48 and records chunk 3
    _case(mss, f"L={seqlen}", 2, 72, seqlen, h0=True)


def test_chunk_states_reverse(mss):
    _case(mss, "reverse", 2, 40, 100, reverse=True, h0=True)


def test_chunk_states_time_split(mss):
    # few channels, long sequence: the forward runs in time segments
    _case(mss, "time-split", 1, 64, 2000, h0=True, a_log="normal")


def test_chunk_states_reverse_time_split(mss):
    _case(mss, "reverse time-split", 1, 64, 1500, reverse=True, h0=True, a_log="normal")


def test_chunk_states_bf16_reverse(mss):
    # an odd length: the element-wise pass for bf16 t-fast vectors in reverse
    _case(mss, "bf16 reverse L=83", 2, 64, 83, io="bf16", reverse=True)


def test_chunk_states_channel_last(mss):
    _case(mss, "bld", 2, 64, 77, layout="bld")


@pytest.mark.parametrize("seqlen", [64, 66])
def test_chunk_states_bf16(mss, seqlen):
    # L = 66: the vector pass stops at 64, so the tail pass records chunk 4
    _case(mss, f"bf16 L={seqlen}", 2, 96, seqlen, io="bf16")


def test_chunk_states_small_dstate(mss):
    _case(mss, "N=5", 2, 40, 70, dstate=5, h0=True)


@pytest.mark.parametrize("shape,reverse", [((2, 72, 100), False), ((2, 72, 100), True),
                                           ((1, 64, 1500), False), ((1, 64, 1500), True),
                                           ((2, 40, 37), False)])
def test_bwd_with_chunk_states(mss, shape, reverse):
    """The backward given the forward's chunk states: against the oracle and
    against the backward that recomputes them."""
    import torch
    batch, dim, seqlen = shape
    dx, init, states = _case(mss, f"bwd {shape} reverse={reverse}", batch, dim, seqlen,
                             reverse=reverse, h0=True, a_log="normal")
    g = torch.Generator().manual_seed(11)
    dout = torch.randn(batch, dim, seqlen, generator=g).to(device())
    dfin = torch.randn(batch, dim, 16, generator=g).to(device())
    args = (dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dout)
    kw = dict(D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=init, dfinal_state=dfin,
              reverse=reverse)
    with_states = mss.selective_scan_bwd(*args, **kw, chunk_states=states)
    without = mss.selective_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    flip = (lambda a: np.ascontiguousarray(to_np(a)[:, :, ::-1])) if reverse else to_np
    ref = oracle.scan_bwd(flip(dx["u"]), flip(dx["delta_raw"]), dx["A_log"], flip(dx["B"]),
                          flip(dx["C"]), flip(dout), D=dx["D"], z=flip(dx["z"]),
                          dt_bias=dx["dt_bias"], h0=init, dfinal=dfin)
    names = {"du": "du", "ddelta_raw": "ddelta_raw", "dB": "dB", "dC": "dC", "dz": "dz",
             "dA_log": "dA_log", "dD": "dD", "ddt_bias": "ddt_bias", "dinitial_state": "dh0"}
    assert set(with_states) == set(without)
    for k, v in with_states.items():
        r = ref[names[k]]
        if reverse and k in ("du", "ddelta_raw", "dB", "dC", "dz"):
            r = r[:, :, ::-1]
        check(f"bwd with chunk states {shape} {k}", to_np(v), r, 1e-4)
        # the two differ only by the rounding of the states: the forward's
        # time segments compose their states in another order
        check(f"bwd with vs without chunk states {shape} {k}", to_np(v), to_np(without[k]), 1e-4)


@pytest.mark.parametrize("shape,layout", [((1, 384, 32768), "bdl"), ((1, 256, 39700), "bld")])
def test_bwd_with_chunk_states_split_aggregates(mss, shape, layout):
    """Few channels, long segments and the forward's chunk states given: the
    backward's segment aggregate pass cuts every segment into two parts (384
    channels x 32768 steps: 64 segments of 32 chunks; 256 channel-last
    channels x 39700 steps: 96 segments of 26 chunks, the last one of 12
    chunks, whose second part is empty, and a ragged last chunk).  Every
    gradient against the oracle."""
    import torch
    batch, dim, seqlen = shape
    note(f"bwd split aggregates: B={batch} D={dim} L={seqlen} {layout}")
    # (the recorded states are checked against oracle prefixes at the shorter
    # lengths above; that check grows with the square of the length)
    dx = to_torch(generate(batch, dim, seqlen, 16, layout, seed=3), device())
    init = torch.randn(batch, dim, 16, generator=torch.Generator().manual_seed(4)).to(device())
    _, states = mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                       D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                       initial_state=init, return_chunk_states=True)
    g = torch.Generator().manual_seed(12)
    dout = torch.randn(batch, dim, seqlen, generator=g)
    if layout == "bld":
        dout = dout.transpose(1, 2).contiguous().transpose(1, 2)
    dout = dout.to(device())
    dfin = torch.randn(batch, dim, 16, generator=g).to(device())
    got = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dout,
                                 D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=init,
                                 dfinal_state=dfin, chunk_states=states)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dout,
                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], h0=init, dfinal=dfin)
    names = {"du": "du", "ddelta_raw": "ddelta_raw", "dB": "dB", "dC": "dC", "dz": "dz",
             "dA_log": "dA_log", "dD": "dD", "ddt_bias": "ddt_bias", "dinitial_state": "dh0"}
    for k, v in got.items():
        check(f"bwd split aggregates {shape} {layout} {k}", to_np(v), ref[names[k]], 1e-4)
