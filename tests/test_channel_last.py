"""Channel-last ([B,L,D]) activations against the oracle: the forward's
vector path there moves whole 128-byte rows shared by the four waves of a
32-channel block, so these cases aim at what that exchange depends on --
channel counts that leave part of the last block empty, time segments (the
aggregate pass too), odd chunk counts per segment, reverse time, both B/C
layouts under channel-last x, bf16 -- and at the chunk states it records.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import generate, to_torch
from util import TOL_BF16, TOL_F32

pytestmark = pytest.mark.gpu

TOL = {"f32": TOL_F32, "bf16": TOL_BF16}


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _relayout(t, unit_axis):
    """The same logical [B, X, L] values stored with unit stride on axis 1
    (channels or states) or axis 2 (time)."""
    if unit_axis == 2:
        return t.contiguous()
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _inputs(batch, dim, seqlen, io, x_axis, bc_axis, seed):
    dx = to_torch(generate(batch, dim, seqlen, 16, "bdl", seed=seed), device(), io)
    for k in ("u", "delta_raw", "z"):
        dx[k] = _relayout(dx[k], x_axis)
    for k in ("B", "C"):
        dx[k] = _relayout(dx[k], bc_axis)
    return dx


def _h0(batch, dim, seed):
    import torch
    return torch.randn(batch, dim, 16, generator=torch.Generator().manual_seed(seed)).to(device())


def _flip(t):
    return None if t is None else t.flip(-1)


def _run(mss, name, dx, io, h0=None, reverse=False, states=False):
    import torch
    res = mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                 D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=h0,
                                 return_final_state=True, reverse=reverse,
                                 return_chunk_states=states)
    torch.cuda.synchronize()
    f = _flip if reverse else (lambda t: t)
    ref_out, ref_fin = oracle.scan_fwd(f(dx["u"]), f(dx["delta_raw"]), dx["A_log"], f(dx["B"]),
                                       f(dx["C"]), D=dx["D"], z=f(dx["z"]), dt_bias=dx["dt_bias"],
                                       h0=h0)
    if reverse:
        ref_out = ref_out[:, :, ::-1]
    check(f"{name} out", to_np(res[0]), ref_out, TOL[io])
    check(f"{name} final", to_np(res[1]), ref_fin, TOL[io])
    return res


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("bc_axis", [1, 2])
@pytest.mark.parametrize("shape", [(1, 200, 3001), (2, 96, 970), (3, 40, 64)])
def test_layouts(mss, io, bc_axis, shape):
    """Channel-last x with n-fast (1) or t-fast (2) B/C.  1x200: 25 tiles in
    7 blocks (three empty waves), time segments; 2x96 over 970 steps: 31
    chunks, an odd count; 3x40: one partly empty block per batch row."""
    batch, dim, seqlen = shape
    note(f"channel-last {io} B/C axis {bc_axis} {shape}")
    dx = _inputs(batch, dim, seqlen, io, 1, bc_axis, seed=31)
    _run(mss, f"channel-last {io} bc{bc_axis} {shape}", dx, io, h0=_h0(batch, dim, 5))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_reverse_time_split(mss, io):
    note(f"channel-last reverse split {io}")
    dx = _inputs(1, 200, 5003, io, 1, 1, seed=32)
    _run(mss, f"channel-last reverse {io}", dx, io, h0=_h0(1, 200, 6), reverse=True)


def test_t_fast_x_with_n_fast_B_C(mss):
    note("t-fast x, n-fast B/C")
    dx = _inputs(2, 72, 1001, "f32", 2, 1, seed=33)
    _run(mss, "t-fast x n-fast B/C", dx, "f32", h0=_h0(2, 72, 7))


@pytest.mark.parametrize("reverse", [False, True])
def test_chunk_states_time_split(mss, reverse):
    """The chunk states a channel-last time-split forward records, against
    oracle prefixes at every 16-step boundary (sampled channels)."""
    note(f"channel-last chunk states reverse={reverse}")
    batch, dim, seqlen = 1, 200, 1500
    dx = _inputs(batch, dim, seqlen, "f32", 1, 1, seed=34)
    h0 = _h0(batch, dim, 8)
    _, _, states = _run(mss, f"channel-last states rev={reverse}", dx, "f32", h0=h0,
                        reverse=reverse, states=True)
    st = to_np(states)
    f = _flip if reverse else (lambda t: t)
    chans = [0, 7, 8, 31, 32, 100, 191, 192, 199]
    sub = {k: f(dx[k])[:, chans] for k in ("u", "delta_raw", "z")}
    for q in range(0, st.shape[0], 7):
        t = 16 * q
        if t == 0:
            ref = to_np(h0)[:, chans]
        else:
            _, ref = oracle.scan_fwd(sub["u"][:, :, :t], sub["delta_raw"][:, :, :t],
                                     dx["A_log"][chans], f(dx["B"])[:, :, :t], f(dx["C"])[:, :, :t],
                                     D=dx["D"][chans], z=sub["z"][:, :, :t],
                                     dt_bias=dx["dt_bias"][chans], h0=h0[:, chans])
        check(f"chunk state {q}", st[q][:, chans, :16], np.asarray(ref), TOL_F32)
