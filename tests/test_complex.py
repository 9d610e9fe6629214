"""GPU parity of the complex-A selective-scan forward against the fp64 complex
oracle (oracle/mss_oracle_cplx.c, pinned in tests/cplx_oracle_pins.py).

Tolerance 1e-4 on max |o - r| / (|r| + rms(r)), the fp32 bar of the real
forward, for the output and for the complex final state: every quantity is
the real forward's recurrence in complex fp32 arithmetic, with the hardware
sin / cos (a few ulp after the reduction to one turn) added to the decay.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import (WORKLOADS, complex_to_torch, generate,
                                             generate_complex, to_torch)

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _cnp(t):
    import torch
    return None if t is None else t.detach().to("cpu", torch.complex128).numpy()


def _run(mss, dx, h0=None, softplus=True, **over):
    q = dict(dx, **over)
    return mss.selective_scan_fwd_complex(q["u"], q["delta_raw"], q["A_log"], q["A_imag"], q["B"],
                                          q["C"], D=q["D"], z=q["z"], dt_bias=q["dt_bias"],
                                          delta_softplus=softplus, initial_state=h0,
                                          return_final_state=True)


def _ref(dx, h0=None, softplus=True, **over):
    q = dict(dx, **over)
    return oracle.scan_fwd_complex(q["u"], q["delta_raw"], q["A_log"], q["A_imag"], _cnp(q["B"]),
                                   _cnp(q["C"]), D=q["D"], z=q["z"], dt_bias=q["dt_bias"],
                                   h0=_cnp(h0), delta_softplus=softplus)


def _h0(batch, dim, dstate, seed=5):
    import torch
    g = torch.Generator().manual_seed(seed)
    re = torch.randn(batch, dim, dstate, generator=g)
    im = torch.randn(batch, dim, dstate, generator=g)
    return torch.complex(re, im).to(device())


def _case(mss, name, batch, dim, seqlen, dstate=16, layout="bdl", h0=False, softplus=True, **over):
    import torch
    note(f"complex {name}: B={batch} D={dim} L={seqlen} N={dstate} {layout} h0={h0} "
         f"softplus={softplus} {sorted(over)}")
    dx = complex_to_torch(generate_complex(batch, dim, seqlen, dstate, layout, seed=13), device())
    for k, v in over.items():
        dx[k] = v
    init = _h0(batch, dim, dstate) if h0 else None
    out, fin = _run(mss, dx, init, softplus)
    torch.cuda.synchronize()
    r_out, r_fin = _ref(dx, init, softplus)
    check(f"complex {name} out", to_np(out), r_out, TOL)
    check(f"complex {name} final", _cnp(fin), r_fin, TOL)
    return dx, out, fin


def test_tiny(mss):
    w = WORKLOADS["tiny"]
    _case(mss, "tiny", w.batch, w.dim, w.seqlen, w.dstate, h0=True)


@pytest.mark.parametrize("seqlen", [1, 7, 32, 33, 100])
def test_ragged_lengths(mss, seqlen):
    _case(mss, f"L={seqlen}", 2, 40, seqlen, h0=True)


@pytest.mark.parametrize("dstate", [1, 5, 13])
def test_small_dstate(mss, dstate):
    _case(mss, f"N={dstate}", 2, 37, 90, dstate, h0=True)


@pytest.mark.parametrize("drop", ["z", "D", "dt_bias"])
def test_optional_inputs(mss, drop):
    _case(mss, f"no {drop}", 2, 48, 70, **{drop: None})


def test_softplus_off(mss):
    import torch
    x = generate_complex(2, 48, 70, 16, seed=13)
    dr = torch.from_numpy(np.abs(x["delta_raw"]) * np.float32(0.5)).to(device())
    bias = torch.from_numpy(np.log1p(np.exp(x["dt_bias"].astype(np.float64))).astype(np.float32))
    _case(mss, "softplus off", 2, 48, 70, softplus=False, delta_raw=dr, dt_bias=bias.to(device()))


def test_time_invariant_B_C(mss):
    import torch
    g = torch.Generator().manual_seed(2)
    base = {k: torch.complex(torch.randn(2, 16, generator=g), torch.randn(2, 16, generator=g))
            .to(device()) for k in ("B", "C")}
    over = {k: base[k][:, :, None].expand(2, 16, 120) for k in ("B", "C")}
    _case(mss, "time-invariant B/C", 2, 40, 120, h0=True, **over)


def test_channel_last(mss):
    _case(mss, "bld", 2, 64, 77, layout="bld", h0=True)


@pytest.mark.parametrize("split", [False, True])
def test_layouts_bitwise_equal(mss, split):
    """The element roles of the load phase follow the layouts (steps fastest
    for unit time stride, channels or states fastest for unit row stride), but
    each (channel, state) lane does the same arithmetic in the same order:
    the four combinations of [B,D,L] / [B,L,D] activations and [B,N,L] /
    [B,L,N] B and C give bitwise equal results, equal to the oracle.  The
    split case (few channels, long sequence) takes the time segments."""
    import torch
    batch, dim, seqlen = (1, 32, 4000) if split else (2, 48, 333)
    note(f"complex layout combinations split={split}")
    dx = complex_to_torch(generate_complex(batch, dim, seqlen, 16, "bdl", seed=17), device())
    init = _h0(batch, dim, 16, seed=9)

    def layout(t, rows_fast):
        return t.transpose(1, 2).contiguous().transpose(1, 2) if rows_fast else t.contiguous()

    res = []
    for x_rows in (False, True):
        for b_rows in (False, True):
            q = dict(dx)
            for k in ("u", "delta_raw", "z"):
                q[k] = layout(dx[k], x_rows)
            for k in ("B", "C"):
                q[k] = layout(dx[k], b_rows)
            res.append(_run(mss, q, init))
    torch.cuda.synchronize()
    for out, fin in res[1:]:
        assert torch.equal(out, res[0][0]) and torch.equal(fin, res[0][1])
    r_out, r_fin = _ref(dx, init)
    check("complex layouts out", to_np(res[0][0]), r_out, TOL)
    check("complex layouts final", _cnp(res[0][1]), r_fin, TOL)


def test_mamba130m_layer_full(mss):
    w = WORKLOADS["mamba130m_layer"]
    _case(mss, "130m layer", w.batch, w.dim, w.seqlen, w.dstate)


def test_mamba2p8b_layer_sampled(mss):
    """The 2.8b layer shape in full on the GPU; a channel sample across every
    batch row against the oracle."""
    import torch
    w = WORKLOADS["mamba2p8b_layer"]
    note("complex 2.8b layer")
    dx = complex_to_torch(generate_complex(w.batch, w.dim, w.seqlen, w.dstate, seed=13), device())
    out, fin = _run(mss, dx)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    chans = np.unique(np.concatenate([[0, 15, 16, w.dim - 1], rng.choice(w.dim, 20, replace=False)]))
    ci = torch.as_tensor(chans, device=device())
    sub = dict(dx, u=dx["u"][:, ci], delta_raw=dx["delta_raw"][:, ci], z=dx["z"][:, ci],
               A_log=dx["A_log"][ci], A_imag=dx["A_imag"][ci], D=dx["D"][ci],
               dt_bias=dx["dt_bias"][ci])
    r_out, r_fin = _ref(sub)
    check("complex 2.8b sampled out", to_np(out[:, ci]), r_out, TOL)
    check("complex 2.8b sampled final", _cnp(fin[:, ci]), r_fin, TOL)


def test_long_sequence_time_split(mss):
    """Few channels, a long ragged sequence: 3 tiles of 16 channels cut into
    hundreds of time segments (aggregates, complex carries, main pass),
    started from an initial state, against the oracle element by element."""
    _case(mss, "time split 48 x 20011", 1, 48, 20011, h0=True)


def test_time_split_channel_last_random_a(mss):
    """The segmented path on channel-last data with A_log ~ N(0, 1) (slow and
    fast decays, so carries reach far), a ragged length and dstate 13."""
    import torch
    x = generate_complex(2, 40, 3001, 13, "bld", seed=21)
    rng = np.random.default_rng(21)
    x["A_log"] = rng.standard_normal(x["A_log"].shape).astype(np.float32)
    dx = complex_to_torch(x, device())
    init = _h0(2, 40, 13)
    note("complex time split, channel-last, random A_log")
    out, fin = _run(mss, dx, init)
    torch.cuda.synchronize()
    r_out, r_fin = _ref(dx, init)
    check("complex split bld random A out", to_np(out), r_out, TOL)
    check("complex split bld random A final", _cnp(fin), r_fin, TOL)


def test_audio_channel_last_sampled(mss):
    """The audio-length channel-last shape (1 x 220500 x 256, 16 tiles, so 64
    time segments) in full on the GPU; sampled channels against the oracle."""
    import torch
    w = WORKLOADS["audio_channel_last"]
    note("complex audio channel-last")
    dx = complex_to_torch(generate_complex(w.batch, w.dim, w.seqlen, w.dstate, w.layout, seed=13),
                          device())
    assert mss.scan_complex_workspace_size(dx["u"], dx["A_log"]) > 0
    out, fin = _run(mss, dx)
    torch.cuda.synchronize()
    chans = np.array([0, 15, 16, 100, 200, w.dim - 1])
    ci = torch.as_tensor(chans, device=device())
    sub = dict(dx, u=dx["u"][:, ci], delta_raw=dx["delta_raw"][:, ci], z=dx["z"][:, ci],
               A_log=dx["A_log"][ci], A_imag=dx["A_imag"][ci], D=dx["D"][ci],
               dt_bias=dx["dt_bias"][ci])
    note(f"complex audio: oracle on {len(chans)} channels")
    r_out, r_fin = _ref(sub)
    check("complex audio sampled out", to_np(out[:, ci]), r_out, TOL)
    check("complex audio sampled final", _cnp(fin[:, ci]), r_fin, TOL)


def test_real_case_matches_real_kernel(mss):
    """Im(A) = 0 with real B, C: the complex kernel and the real forward kernel
    (separate code) agree."""
    import torch
    x = generate(2, 72, 150, 16, seed=9)
    dx = to_torch(x, device(), "f32")
    zero = torch.zeros_like(dx["A_log"])
    Bc = torch.complex(dx["B"], torch.zeros_like(dx["B"]))
    Cc = torch.complex(dx["C"], torch.zeros_like(dx["C"]))
    note("complex vs real kernel")
    out_c, fin_c = mss.selective_scan_fwd_complex(dx["u"], dx["delta_raw"], dx["A_log"], zero, Bc,
                                                  Cc, D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                                  return_final_state=True)
    out_r, fin_r = mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                          return_final_state=True)
    torch.cuda.synchronize()
    check("complex vs real out", to_np(out_c), to_np(out_r), 1e-5)
    check("complex vs real final", to_np(fin_c.real), to_np(fin_r), 1e-5)
    assert float(fin_c.imag.abs().max()) == 0.0


def test_run_twice_bitwise(mss):
    import torch
    dx = complex_to_torch(generate_complex(2, 40, 100, 16, seed=4), device())
    h0 = _h0(2, 40, 16)
    a = _run(mss, dx, h0)
    b = _run(mss, dx, h0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
