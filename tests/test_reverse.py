"""GPU parity of the reverse-time scan (the second direction of a bidirectional
layer) against the fp64 oracle run on the time-reversed sequence.

The reverse scan on buffers x is by definition the forward scan on x with its
time axis reversed, with the outputs reversed back: out_rev[t] = flip(scan(
flip(x)))[t], and the final state is the state after storage step 0.  The
gradients of the reverse backward are likewise the flipped gradients of the
flipped problem.  Tolerances as in test_parity.py / test_bwd_parity.py.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import generate, to_torch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TIME_AXIS = {"u": 2, "delta_raw": 2, "z": 2, "B": 2, "C": 2, "dout": 2}


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _flip(a):
    return None if a is None else np.ascontiguousarray(to_np(a)[:, :, ::-1])


def _fwd_case(mss, name, batch, dim, seqlen, layout="bdl", io="f32", h0=False, a_log="ladder"):
    import torch
    note(f"reverse fwd {name}: B={batch} D={dim} L={seqlen} {layout} {io} h0={h0}")
    x = generate(batch, dim, seqlen, 16, layout, seed=21, a_log=a_log)
    dx = to_torch(x, device(), io)
    init = torch.randn(batch, dim, 16, generator=torch.Generator().manual_seed(2)).to(device()) \
        if h0 else None
    out, fin = mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                      D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                      initial_state=init, return_final_state=True, reverse=True)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.scan_fwd(_flip(dx["u"]), _flip(dx["delta_raw"]), dx["A_log"],
                                       _flip(dx["B"]), _flip(dx["C"]), D=dx["D"], z=_flip(dx["z"]),
                                       dt_bias=dx["dt_bias"], h0=init)
    check(f"reverse {name} out", to_np(out), ref_out[:, :, ::-1], TOL[io])
    check(f"reverse {name} final", to_np(fin), ref_fin, TOL[io])


@pytest.mark.parametrize("seqlen", [1, 7, 32, 33, 2049])
def test_reverse_bdl(mss, seqlen):
    _fwd_case(mss, f"bdl L={seqlen}", 2, 72, seqlen, h0=True)


@pytest.mark.parametrize("seqlen", [5, 300])
def test_reverse_channel_last(mss, seqlen):
    _fwd_case(mss, f"bld L={seqlen}", 2, 64, seqlen, layout="bld")


@pytest.mark.parametrize("seqlen", [200, 201])
def test_reverse_bf16(mss, seqlen):
    # an odd length takes the element-wise path for bf16 t-fast vectors
    _fwd_case(mss, f"bf16 L={seqlen}", 2, 96, seqlen, io="bf16")


def test_reverse_time_split(mss):
    _fwd_case(mss, "time-split", 1, 64, 20000, h0=True, a_log="normal")


def test_reverse_mamba130m_layer(mss):
    _fwd_case(mss, "130m layer", 1, 1536, 2048)


def test_bidirectional_sum(mss):
    """A bidirectional layer's two directions on one set of buffers: the forward
    plus the reverse scan equals the oracle's forward plus its flipped-input run."""
    import torch
    x = generate(1, 128, 500, 16, seed=8)
    dx = to_torch(x, device(), "f32")
    args = (dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"])
    kw = dict(D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"])
    note("bidirectional sum")
    both = mss.selective_scan_fwd(*args, **kw) + mss.selective_scan_fwd(*args, **kw, reverse=True)
    torch.cuda.synchronize()
    f, _ = oracle.scan_fwd(*[to_np(a) for a in args], D=x["D"], z=x["z"], dt_bias=x["dt_bias"])
    r, _ = oracle.scan_fwd(_flip(dx["u"]), _flip(dx["delta_raw"]), x["A_log"], _flip(dx["B"]),
                           _flip(dx["C"]), D=x["D"], z=_flip(dx["z"]), dt_bias=x["dt_bias"])
    check("bidirectional sum", to_np(both), f + r[:, :, ::-1], 1e-4)


@pytest.mark.parametrize("shape,layout,io", [
    ((2, 72, 100), "bdl", "f32"), ((1, 64, 1500), "bdl", "f32"), ((1, 40, 1500), "bld", "f32"),
    ((2, 48, 333), "bld", "f32"),
    # bf16: step pairs and 4-step vectors, with and without time segments, and
    # an odd length (element by element)
    ((2, 72, 100), "bdl", "bf16"), ((1, 64, 1500), "bdl", "bf16"), ((1, 40, 1501), "bdl", "bf16"),
    ((1, 64, 998), "bld", "bf16")])
def test_reverse_backward(mss, shape, layout, io):
    import torch
    batch, dim, seqlen = shape
    note(f"reverse bwd {shape} {layout} {io}")
    x = generate(batch, dim, seqlen, 16, layout, seed=23, a_log="normal")
    dx = to_torch(x, device(), io)
    g = torch.Generator().manual_seed(5)
    dout = torch.randn(batch, dim, seqlen, generator=g)
    if layout == "bld":
        dout = dout.transpose(1, 2).contiguous().transpose(1, 2)
    dout = dout.to(device=device(), dtype=dx["u"].dtype)
    h0 = torch.randn(batch, dim, 16, generator=g).to(device())
    dfin = torch.randn(batch, dim, 16, generator=g).to(device())
    got = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dout,
                                 D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=h0,
                                 dfinal_state=dfin, reverse=True)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(_flip(dx["u"]), _flip(dx["delta_raw"]), dx["A_log"], _flip(dx["B"]),
                          _flip(dx["C"]), _flip(dout), D=dx["D"], z=_flip(dx["z"]),
                          dt_bias=dx["dt_bias"], h0=h0, dfinal=dfin)
    names = {"du": "du", "ddelta_raw": "ddelta_raw", "dB": "dB", "dC": "dC", "dz": "dz",
             "dA_log": "dA_log", "dD": "dD", "ddt_bias": "ddt_bias", "dinitial_state": "dh0"}
    for k, v in got.items():
        r = ref[names[k]]
        if k in ("du", "ddelta_raw", "dB", "dC", "dz"):
            r = r[:, :, ::-1]
        check(f"reverse bwd {shape} {io} {k}", to_np(v), r, TOL[io])
