"""GPU parity of the causal depthwise conv1d (+ SiLU) and its decode step
against the fp64 oracle on seeded synthetic inputs.

Tolerances (error metric: max |o - r| / (|r| + rms(r))):
  fp32 I/O 1e-5: at most four fp32 FMAs and a SiLU built from the hardware
      exp2 and reciprocal (each within a few ulp) separate the result from the
      exact value, i.e. a few 1e-7 of the output's scale;
  bf16 I/O 4e-3: the oracle reads the same rounded inputs, so the error is the
      rounding of the output to bf16, at most 2^-9 relative, plus the fp32
      error above.
The windows are copies of input samples and must match exactly.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import conv_to_torch, generate_conv

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 4e-3}


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _case(mss, name, batch, dim, seqlen, width=4, layout="bld", io="f32", seed=0,
          silu=True, bias=True, window=False, view=None):
    import torch
    note(f"conv {name}: B={batch} D={dim} L={seqlen} W={width} {layout} {io} silu={silu} "
         f"bias={bias} window={window} view={view}")
    x = generate_conv(batch, dim, seqlen, width, layout, seed=seed)
    dx = conv_to_torch(x, device(), io)
    xt = dx["x"]
    if view == "offset":
        # a view one element into a larger buffer: vector loads would be misaligned
        big = torch.empty(batch, dim, seqlen + 1, dtype=xt.dtype, device=xt.device)
        big[:, :, 1:] = xt
        xt = big[:, :, 1:]
    elif view == "padded":
        # rows padded to a whole number of 16-byte vectors: the vector path
        # with a partial vector at the end of every row
        pad = (-seqlen) % 8 + 8
        big = torch.zeros(batch, dim, seqlen + pad, dtype=xt.dtype, device=xt.device)
        big[:, :, :seqlen] = xt
        xt = big[:, :, :seqlen]
    elif view == "strided":
        # every other channel of a wider buffer: no unit-stride axis for d
        big = torch.zeros(batch, seqlen, 2 * dim, dtype=xt.dtype, device=xt.device)
        big[:, :, ::2] = xt.transpose(1, 2)
        xt = big[:, :, ::2].transpose(1, 2)
    init = dx["window"] if window else None
    out, fin = mss.causal_conv1d_fwd(xt, dx["weight"], dx["bias"] if bias else None,
                                     activation="silu" if silu else None, initial_state=init,
                                     return_final_state=True)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.conv1d_fwd(dx["x"], dx["weight"], dx["bias"] if bias else None,
                                         init, silu=silu)
    check(f"conv {name} out", to_np(out), ref_out, TOL[io])
    assert np.array_equal(to_np(fin), ref_fin), f"conv {name}: final window differs"


def test_audio_channel_last_full(mss):
    # the SpeechLens fixture length: 5 s at 44.1 kHz, 256 channels, [B, L, D]
    _case(mss, "audio", 1, 256, 220500)


def test_mamba130m_shape_both_layouts(mss):
    _case(mss, "130m bld", 1, 1536, 2048, layout="bld")
    _case(mss, "130m bdl", 1, 1536, 2048, layout="bdl")


@pytest.mark.parametrize("layout", ["bld", "bdl"])
@pytest.mark.parametrize("seqlen", [1, 2, 3, 5, 63, 1023, 1025, 4097])
def test_ragged_lengths(mss, layout, seqlen):
    _case(mss, f"L={seqlen}", 2, 264, seqlen, layout=layout, window=True)


@pytest.mark.parametrize("width", [1, 2, 3])
@pytest.mark.parametrize("layout", ["bld", "bdl"])
def test_widths(mss, width, layout):
    _case(mss, f"W={width}", 2, 260, 300, width=width, layout=layout, window=True)


@pytest.mark.parametrize("flags", [dict(silu=False), dict(bias=False), dict(window=True),
                                   dict(silu=False, bias=False, window=True)])
@pytest.mark.parametrize("layout", ["bld", "bdl"])
def test_options(mss, flags, layout):
    _case(mss, f"opts {flags}", 3, 128, 777, layout=layout, **flags)


@pytest.mark.parametrize("layout", ["bld", "bdl"])
def test_bf16(mss, layout):
    _case(mss, "bf16", 2, 512, 3000, layout=layout, io="bf16", window=True)


@pytest.mark.parametrize("dim", [1, 6, 300])
def test_channel_counts(mss, dim):
    # 1 and 6 are not whole vectors of channels (element-wise path); 300 leaves
    # part of the last 256-channel group empty
    _case(mss, f"D={dim}", 2, dim, 513, window=True)


@pytest.mark.parametrize("view", ["offset", "strided"])
def test_views(mss, view):
    _case(mss, f"view {view}", 2, 96, 500, view=view, window=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("seqlen", [1, 5, 2045, 2049, 4103])
def test_padded_rows(mss, io, seqlen):
    _case(mss, f"padded L={seqlen}", 2, 40, seqlen, layout="bdl", io=io, view="padded",
          window=True)


def test_mamba2p8b_shape_sampled(mss):
    import torch
    batch, dim, seqlen = 8, 5120, 4096
    note(f"conv 2.8b shape: B={batch} D={dim} L={seqlen} bld f32")
    x = generate_conv(batch, dim, seqlen, 4, "bld", seed=3)
    dx = conv_to_torch(x, device(), "f32")
    out, fin = mss.causal_conv1d_fwd(dx["x"], dx["weight"], dx["bias"], return_final_state=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    chans = sorted({(0, 0), (batch - 1, dim - 1)} |
                   {(int(rng.integers(batch)), int(rng.integers(dim))) for _ in range(62)})
    got = np.stack([to_np(out[b, d]) for b, d in chans])
    ref = np.stack([oracle.conv1d_fwd(x["x"][b:b + 1, d:d + 1], x["weight"][d:d + 1],
                                      x["bias"][d:d + 1])[0][0, 0] for b, d in chans])
    check("conv 2.8b shape sampled out", got, ref, TOL["f32"])
    got_fin = np.stack([to_np(fin[b, d]) for b, d in chans])
    ref_fin = np.stack([x["x"][b, d, -3:] for b, d in chans]).astype(np.float64)
    assert np.array_equal(got_fin, ref_fin)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("width", [1, 4])
def test_prefill_then_decode(mss, io, width):
    """Conv over L steps with the window exported, then 64 decode steps: every
    output and the final window equal one oracle conv over L + 64 steps."""
    import torch
    batch, dim, L, extra = 2, 384, 1000, 64
    note(f"conv hand-off {io} W={width}: L={L} + {extra} steps")
    x = generate_conv(batch, dim, L + extra, width, "bld", seed=5)
    dx = conv_to_torch(x, device(), io)
    out, win = mss.causal_conv1d_fwd(dx["x"][:, :, :L], dx["weight"], dx["bias"],
                                     return_final_state=True)
    outs = []
    for t in range(L, L + extra):
        outs.append(mss.causal_conv1d_update(win, dx["x"][:, :, t], dx["weight"], dx["bias"]))
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.conv1d_fwd(dx["x"], dx["weight"], dx["bias"])
    check(f"conv hand-off {io} prefill", to_np(out), ref_out[:, :, :L], TOL[io])
    got = np.stack([to_np(o) for o in outs], axis=2)
    check(f"conv hand-off {io} decode", got, ref_out[:, :, L:], TOL[io])
    assert np.array_equal(to_np(win), ref_fin)


def test_decode_step_no_silu_strided(mss):
    import torch
    batch, dim, width = 3, 200, 4
    note("conv decode step: strided x/out, no activation")
    x = generate_conv(batch, dim, 1, width, "bdl", seed=9)
    dx = conv_to_torch(x, device(), "f32")
    big = torch.randn(batch, 2 * dim, device=device())
    xs = big[:, ::2]
    state = dx["window"].clone()
    out = torch.empty(batch, 2 * dim, device=device())[:, 1::2]
    mss.causal_conv1d_update(state, xs, dx["weight"], dx["bias"], activation=None, out=out)
    torch.cuda.synchronize()
    ref, ref_state = oracle.conv1d_update(dx["window"], xs, dx["weight"], dx["bias"], silu=False)
    check("conv decode strided", to_np(out), ref, TOL["f32"])
    assert np.array_equal(to_np(state), ref_state)
