"""GPU parity past the 32-bit wrap points of element counts and byte offsets.

A [2, 4096, 280000] float32 tensor holds 2.29e9 elements (more than 2^31) in
9.2 GB (more than 2^33 bytes), so the channels of the second batch row lie past
every 32-bit wrap point of both.  The kernels address memory through 64-bit
tile or row bases plus 32-bit offsets inside a tile; these tests run that
arithmetic where a 32-bit product would wrap: the scan forward in both layouts
(with time segments: the shape has 1024 channel tiles), the backward, the
complex-A forward and the conv.  Sampled channels, the first and last of each
batch row among them, are compared over their whole sequences with the oracle
at the fp32 tolerance.
Inputs are drawn on the device (``generate_device``: the workload recipe with
torch's generator).  Device memory: about 40 GB for the forward, the complex
forward and the conv, 85 GB for the backward, released after each test.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import generate_device

pytestmark = pytest.mark.gpu

BATCH, DIM, SEQLEN, DSTATE = 2, 4096, 280000, 16
CHANNELS = [(0, 0), (0, DIM - 1), (1, 0), (1, DIM // 2 - 1), (1, DIM - 1)]
TOL = 1e-4


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


@pytest.fixture
def fresh_memory():
    import torch
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_shape_is_past_the_wrap_points():
    assert BATCH * DIM * SEQLEN > 2 ** 31
    assert (BATCH * DIM * SEQLEN - 1) * 4 > 2 ** 33
    # the last sampled channel starts past 2^33 bytes in [B, D, L] storage
    b, d = CHANNELS[-1]
    assert (b * DIM + d) * SEQLEN * 4 > 2 ** 33


@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_forward_past_32bit_offsets(mss, fresh_memory, layout):
    import torch
    note(f"large forward: B={BATCH} D={DIM} L={SEQLEN} N={DSTATE} {layout} f32")
    x = generate_device(BATCH, DIM, SEQLEN, DSTATE, layout, seed=3, device=device())
    out, fin = mss.selective_scan_fwd(x["u"], x["delta_raw"], x["A_log"], x["B"], x["C"],
                                      D=x["D"], z=x["z"], dt_bias=x["dt_bias"],
                                      return_final_state=True)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.scan_channels(x, CHANNELS)
    got_out = np.stack([to_np(out[b, d]) for b, d in CHANNELS])
    got_fin = np.stack([to_np(fin[b, d]) for b, d in CHANNELS])
    check(f"large forward {layout} out", got_out, ref_out, TOL)
    check(f"large forward {layout} final_state", got_fin, ref_fin, TOL)


def test_backward_past_32bit_offsets(mss, fresh_memory):
    """du, ddelta_raw and dz of the sampled channels in both batch rows, and
    dA_log, dD, ddt_bias of those channels (sums over both rows).  dB and dC sum
    over all 4096 channels, beyond what the oracle computes here; smaller
    shapes check them."""
    import torch
    note(f"large backward: B={BATCH} D={DIM} L={SEQLEN} N={DSTATE} bdl f32")
    x = generate_device(BATCH, DIM, SEQLEN, DSTATE, "bdl", seed=4, device=device())
    g = torch.Generator(device=device()).manual_seed(44)
    dout = torch.randn(BATCH, DIM, SEQLEN, generator=g, device=device())
    got = mss.selective_scan_bwd(x["u"], x["delta_raw"], x["A_log"], x["B"], x["C"], dout,
                                 D=x["D"], z=x["z"], dt_bias=x["dt_bias"])
    torch.cuda.synchronize()
    chans = sorted({d for _, d in CHANNELS})
    ci = torch.as_tensor(chans, device=device())
    ref = oracle.scan_bwd(x["u"][:, ci], x["delta_raw"][:, ci], x["A_log"][ci], x["B"], x["C"],
                          dout[:, ci], D=x["D"][ci], z=x["z"][:, ci], dt_bias=x["dt_bias"][ci])
    for k in ("du", "ddelta_raw", "dz"):
        check(f"large backward {k}", to_np(got[k][:, ci]), ref[k], TOL)
    for k in ("dA_log", "dD", "ddt_bias"):
        check(f"large backward {k}", to_np(got[k][ci]), ref[k], TOL)


@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_complex_forward_past_32bit_offsets(mss, fresh_memory, layout):
    """Complex B and C with unit complex variance and A_imag = pi n, as the
    complex workload recipe has them, drawn on the device."""
    import torch
    note(f"large complex forward: B={BATCH} D={DIM} L={SEQLEN} N={DSTATE} {layout} f32")
    x = generate_device(BATCH, DIM, SEQLEN, DSTATE, layout, seed=6, device=device())
    g = torch.Generator(device=device()).manual_seed(66)
    half = 0.5 ** 0.5
    for k in ("B", "C"):
        shape = (BATCH, DSTATE, SEQLEN) if layout == "bdl" else (BATCH, SEQLEN, DSTATE)
        re = torch.randn(shape, generator=g, device=device()) * half
        im = torch.randn(shape, generator=g, device=device()) * half
        c = torch.complex(re, im)
        x[k] = c if layout == "bdl" else c.transpose(1, 2)
    a_imag = torch.pi * torch.arange(DSTATE, device=device(), dtype=torch.float32)
    x["A_imag"] = a_imag.expand(DIM, DSTATE).contiguous()
    out, fin = mss.selective_scan_fwd_complex(x["u"], x["delta_raw"], x["A_log"], x["A_imag"],
                                              x["B"], x["C"], D=x["D"], z=x["z"],
                                              dt_bias=x["dt_bias"], return_final_state=True)
    torch.cuda.synchronize()
    for b in range(BATCH):
        ds = [d for bb, d in CHANNELS if bb == b]
        ci = torch.as_tensor(ds, device=device())
        row = slice(b, b + 1)
        cnp = lambda t: t.detach().to("cpu", torch.complex128).numpy()  # noqa: E731
        r_out, r_fin = oracle.scan_fwd_complex(
            x["u"][row, ci], x["delta_raw"][row, ci], x["A_log"][ci], x["A_imag"][ci],
            cnp(x["B"][row]), cnp(x["C"][row]), D=x["D"][ci], z=x["z"][row, ci],
            dt_bias=x["dt_bias"][ci])
        check(f"large complex {layout} row {b} out", to_np(out[row, ci]), r_out, TOL)
        check(f"large complex {layout} row {b} final", cnp(fin[row, ci]), r_fin, TOL)


@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_conv_past_32bit_offsets(mss, fresh_memory, layout):
    import torch
    note(f"large conv1d: B={BATCH} D={DIM} L={SEQLEN} width 4 {layout} f32")
    g = torch.Generator(device=device()).manual_seed(5)
    shape = (BATCH, DIM, SEQLEN) if layout == "bdl" else (BATCH, SEQLEN, DIM)
    xs = torch.randn(shape, generator=g, device=device())
    x = xs if layout == "bdl" else xs.transpose(1, 2)
    bound = 0.5  # 1 / sqrt(width)
    w = (torch.rand(DIM, 4, generator=g, device=device()) * 2 - 1) * bound
    bias = (torch.rand(DIM, generator=g, device=device()) * 2 - 1) * bound
    out = mss.causal_conv1d_fwd(x, w, bias)
    torch.cuda.synchronize()
    for b in range(BATCH):
        ds = [d for bb, d in CHANNELS if bb == b]
        ci = torch.as_tensor(ds, device=device())
        ref, _ = oracle.conv1d_fwd(x[b:b + 1, ci], w[ci], bias[ci])
        check(f"large conv {layout} row {b}", to_np(out[b:b + 1, ci]), ref, TOL)
