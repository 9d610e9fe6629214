"""Seeded synthetic inputs for the selective-scan forward and state update.

This module holds only input generation: it draws random tensors and builds
the parameter tensors of the workloads below.  It performs none of the scan's
arithmetic, and it is the one module that both the HIP path's callers and the
fp64 oracle's callers share.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order, each
in its storage shape, in float32):
    u ~ N(0, 1);  delta_raw ~ N(0, 0.1^2);  z ~ N(0, 1);  B ~ N(0, 1);  C ~ N(0, 1)
then per channel d: dt_d = exp(U(log 1e-3, log 0.1)) and
dt_bias_d = log(expm1(dt_d)) (the value whose softplus is dt_d), float32;
A_log[d, n] = log(n + 1); D = 1.
Storage shapes: u, delta_raw, z are [B, D, L] and B, C are [B, N, L] in the
"bdl" layout; [B, L, D] and [B, L, N] in the "bld" (channel-last) layout.
Arrays are returned in logical index order (u as [b, d, t], B as [b, n, t]),
as views over the storage layout.  bfloat16 copies are made with torch's
round-to-nearest-even conversion; callers hand the same rounded values to
both the GPU and the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    layout: str = "bdl"          # "bdl" ([B,D,L] / [B,N,L]) or "bld" ([B,L,D] / [B,L,N])
    decode_steps: int = 0        # extra timesteps drawn for a decode hand-off

    @property
    def elems(self) -> int:
        return self.batch * self.dim * self.seqlen


# The five workload shapes: a tiny scan, a mamba-130m-shaped layer, a
# mamba-2.8b-shaped layer, a 32k-token sequence followed by 64 decode steps,
# and a channel-last audio-length sequence (5 s at 44.1 kHz).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 256, 16),
    "mamba130m_layer": Workload("mamba130m_layer", 1, 1536, 2048, 16),
    "mamba2p8b_layer": Workload("mamba2p8b_layer", 8, 5120, 4096, 16),
    "long_handoff": Workload("long_handoff", 1, 1536, 32768, 16, decode_steps=64),
    "audio_channel_last": Workload("audio_channel_last", 1, 256, 220500, 16, layout="bld"),
}


def generate(batch: int, dim: int, seqlen: int, dstate: int, layout: str = "bdl",
             seed: int = 0, a_log: str = "ladder", d_skip: str = "ones") -> dict:
    """Draw one problem.  Returns numpy float32 arrays in logical index order.

    a_log="ladder" gives A_log[d, n] = log(n + 1); a_log="normal" draws
    A_log ~ N(0, 1) instead (after everything else, same stream).
    d_skip="ones" gives D = 1; "normal" draws D ~ N(0, 1); "zeros" gives D = 0.
    """
    if layout not in ("bdl", "bld"):
        raise ValueError("layout must be 'bdl' or 'bld'")
    rng = np.random.default_rng(seed)
    f32 = np.float32
    if layout == "bdl":
        x_shape, bc_shape = (batch, dim, seqlen), (batch, dstate, seqlen)
    else:
        x_shape, bc_shape = (batch, seqlen, dim), (batch, seqlen, dstate)

    def draw(shape, scale=1.0):
        a = rng.standard_normal(shape, dtype=f32)
        if scale != 1.0:
            a *= f32(scale)
        return a

    u = draw(x_shape)
    delta_raw = draw(x_shape, 0.1)
    z = draw(x_shape)
    Bm = draw(bc_shape)
    Cm = draw(bc_shape)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=dim))
    dt_bias = np.log(np.expm1(dt)).astype(f32)
    if a_log == "ladder":
        A_log = np.tile(np.log(np.arange(1, dstate + 1, dtype=np.float64)), (dim, 1)).astype(f32)
    elif a_log == "normal":
        A_log = rng.standard_normal((dim, dstate)).astype(f32)
    else:
        raise ValueError(a_log)
    if d_skip == "ones":
        D = np.ones(dim, dtype=f32)
    elif d_skip == "normal":
        D = rng.standard_normal(dim).astype(f32)
    elif d_skip == "zeros":
        D = np.zeros(dim, dtype=f32)
    else:
        raise ValueError(d_skip)

    if layout == "bld":
        u, delta_raw, z = (a.transpose(0, 2, 1) for a in (u, delta_raw, z))
        Bm, Cm = (a.transpose(0, 2, 1) for a in (Bm, Cm))
    return {"u": u, "delta_raw": delta_raw, "z": z, "B": Bm, "C": Cm,
            "A_log": A_log, "D": D, "dt_bias": dt_bias, "layout": layout}


def generate_device(batch: int, dim: int, seqlen: int, dstate: int, layout: str = "bdl",
                    seed: int = 0, device="cuda") -> dict:
    """The recipe of ``generate`` drawn on ``device`` with torch's generator,
    for problems too large to draw on the host and copy over (tensors of many
    GiB).  The distributions are the same; the random stream is torch's
    (u, delta_raw, z, B, C drawn in that order from one generator seeded with
    ``seed``), not numpy's.  The small per-channel parameters (dt_bias,
    A_log = log(n + 1), D = 1) come from ``generate``'s own rules, dt from a
    numpy stream seeded with ``seed``.  Returns float32 torch tensors in
    logical index order, as views over the storage layout."""
    import torch

    if layout not in ("bdl", "bld"):
        raise ValueError("layout must be 'bdl' or 'bld'")
    g = torch.Generator(device=device).manual_seed(seed)
    if layout == "bdl":
        x_shape, bc_shape = (batch, dim, seqlen), (batch, dstate, seqlen)
    else:
        x_shape, bc_shape = (batch, seqlen, dim), (batch, seqlen, dstate)

    def draw(shape, scale=1.0):
        a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            a.mul_(scale)
        return a if layout == "bdl" else a.transpose(1, 2)

    out = {"u": draw(x_shape), "delta_raw": draw(x_shape, 0.1), "z": draw(x_shape),
           "B": draw(bc_shape), "C": draw(bc_shape)}
    rng = np.random.default_rng(seed)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(0.1), size=dim))
    out["dt_bias"] = torch.from_numpy(np.log(np.expm1(dt)).astype(np.float32)).to(device)
    a_log = np.tile(np.log(np.arange(1, dstate + 1, dtype=np.float64)), (dim, 1))
    out["A_log"] = torch.from_numpy(a_log.astype(np.float32)).to(device)
    out["D"] = torch.ones(dim, device=device, dtype=torch.float32)
    return out


def softplus_range_delta(batch: int, dim: int, seqlen: int, seed: int = 0,
                         big_bias: bool = False) -> tuple:
    """(delta_raw [batch, dim, seqlen], dt_bias [dim]) float32 whose sum
    x = delta_raw + dt_bias covers the softplus argument far beyond the usual
    draw: a uniform grid over [-40, 40] (step 0.5), a dense grid across
    [19.5, 20.5] (step 0.01, the region of the x > 20 shortcut some kernels
    take) and U(30, 45) values, repeated along time in a random order per
    channel.  dt_bias is 0, or with ``big_bias`` 25 on every second channel,
    whose delta_raw is then the grid minus 25.
    """
    rng = np.random.default_rng(seed + 2_000_003)
    grid = np.concatenate([np.arange(-80, 81) * 0.5, 19.5 + 0.01 * np.arange(101),
                           rng.uniform(30.0, 45.0, 40)])
    reps = -(-seqlen // grid.size)
    xs = np.empty((batch, dim, seqlen), dtype=np.float64)
    for b in range(batch):
        for d in range(dim):
            xs[b, d] = rng.permutation(np.tile(grid, reps))[:seqlen]
    dt_bias = np.zeros(dim, dtype=np.float32)
    if big_bias:
        dt_bias[1::2] = np.float32(25.0)
    delta_raw = (xs - dt_bias[None, :, None].astype(np.float64)).astype(np.float32)
    return delta_raw, dt_bias


def generate_workload(w: Workload, seed: int = 0, **kw) -> dict:
    """Draw a named workload (with its extra decode timesteps, if any)."""
    return generate(w.batch, w.dim, w.seqlen + w.decode_steps, w.dstate, w.layout,
                    seed=seed, **kw)


def generate_complex(batch: int, dim: int, seqlen: int, dstate: int, layout: str = "bdl",
                     seed: int = 0) -> dict:
    """A complex-A problem: the real problem of ``generate`` (u, delta_raw, z,
    A_log = log(n + 1), D = 1, dt_bias) with A_imag[d, n] = pi n (the
    S4D-Lin rotation ladder) and complex B, C whose real and imaginary parts
    are independent N(0, 1/2) (unit complex variance), as complex64 in logical
    index order [batch, dstate, seqlen]."""
    x = generate(batch, dim, seqlen, dstate, layout, seed=seed)
    rng = np.random.default_rng(seed + 1_000_003)
    shape = (batch, dstate, seqlen) if layout == "bdl" else (batch, seqlen, dstate)
    half = np.float32(np.sqrt(0.5))
    for k in ("B", "C"):
        re = rng.standard_normal(shape, dtype=np.float32) * half
        im = rng.standard_normal(shape, dtype=np.float32) * half
        c = (re + 1j * im).astype(np.complex64)
        x[k] = c if layout == "bdl" else c.transpose(0, 2, 1)
    x["A_imag"] = np.tile(np.float32(np.pi) * np.arange(dstate, dtype=np.float32), (dim, 1))
    return x


def complex_to_torch(inputs: dict, device) -> dict:
    """Move a complex-A problem to ``device`` (fp32 activations, complex64 B
    and C), keeping the storage layout as to_torch does."""
    import torch

    out = {"layout": inputs["layout"]}
    for k, dt in (("u", torch.float32), ("delta_raw", torch.float32), ("z", torch.float32),
                  ("B", torch.complex64), ("C", torch.complex64)):
        a = inputs[k]
        if inputs["layout"] == "bld":
            t = torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1)))
            out[k] = t.to(device=device, dtype=dt).transpose(1, 2)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
    for k in ("A_log", "A_imag", "D", "dt_bias"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inputs[k])).to(device)
    return out


def complex_algorithmic_bytes(batch, dim, seqlen, dstate, final_state=True) -> int:
    """Bytes a complex-A forward must move: u, delta_raw, z read and out
    written (fp32), B and C read (complex64), the [D, N] parameters and D,
    dt_bias, and the complex final state."""
    n = 4 * batch * dim * seqlen * 4 + 2 * batch * dstate * seqlen * 8
    n += 2 * dim * dstate * 4 + 2 * dim * 4
    if final_state:
        n += batch * dim * dstate * 8
    return n


def to_torch(inputs: dict, device, io_dtype: str = "f32") -> dict:
    """Move a generated problem to ``device``.

    u, delta_raw, z, B and C take ``io_dtype`` ("f32" or "bf16", converted with
    round-to-nearest-even); A_log, D and dt_bias stay float32.  The storage
    layout is kept: logical-order views over it are returned.
    """
    import torch

    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[io_dtype]
    out = {"layout": inputs["layout"]}
    for k in ("u", "delta_raw", "z", "B", "C"):
        a = inputs[k]
        if inputs["layout"] == "bld":
            t = torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1)))
            t = t.to(device=device, dtype=dt).transpose(1, 2)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
        out[k] = t
    for k in ("A_log", "D", "dt_bias"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inputs[k])).to(device)
    return out


def slice_time(inputs: dict, start: int, stop: int) -> dict:
    """Sub-range of timesteps [start, stop) of a problem (views, any backend)."""
    out = dict(inputs)
    for k in ("u", "delta_raw", "z", "B", "C"):
        out[k] = inputs[k][:, :, start:stop]
    return out


def algorithmic_bytes(batch: int, dim: int, seqlen: int, dstate: int, io_bytes: int,
                      final_state: bool = False, has_z: bool = True, has_D: bool = True,
                      has_dt_bias: bool = True, bc_time_invariant: bool = False) -> int:
    """Bytes the forward must move: each input read once, each output written once.
    Time-invariant B and C are one [batch, dstate] value each."""
    per_bdl = 3 + int(has_z)          # u, delta_raw, out (+ z)
    n = batch * dim * seqlen * per_bdl * io_bytes
    n += 2 * batch * (1 if bc_time_invariant else seqlen) * dstate * io_bytes   # B, C
    n += dim * dstate * 4                          # A_log
    n += dim * 4 * (int(has_D) + int(has_dt_bias))
    if final_state:
        n += batch * dim * dstate * 4
    return n


def generate_conv(batch: int, dim: int, seqlen: int, width: int = 4, layout: str = "bld",
                  seed: int = 0) -> dict:
    """Draw one conv1d problem.  Returns numpy float32 arrays in logical order.

    One ``numpy.random.default_rng(seed)`` stream, in this order: x ~ N(0, 1) in
    its storage shape ([B, L, D] for "bld", [B, D, L] for "bdl"); weight [D, W]
    and bias [D] ~ U(-1/sqrt(W), 1/sqrt(W)) (the default initialisation of a
    framework Conv1d with W inputs per output); a carried window [B, D, W-1]
    ~ N(0, 1).  x is returned as a [b, d, t] view over its storage.
    """
    if layout not in ("bdl", "bld"):
        raise ValueError("layout must be 'bdl' or 'bld'")
    rng = np.random.default_rng(seed)
    f32 = np.float32
    shape = (batch, dim, seqlen) if layout == "bdl" else (batch, seqlen, dim)
    x = rng.standard_normal(shape, dtype=f32)
    bound = 1.0 / np.sqrt(width)
    weight = rng.uniform(-bound, bound, size=(dim, width)).astype(f32)
    bias = rng.uniform(-bound, bound, size=dim).astype(f32)
    window = rng.standard_normal((batch, dim, width - 1), dtype=f32)
    if layout == "bld":
        x = x.transpose(0, 2, 1)
    return {"x": x, "weight": weight, "bias": bias, "window": window, "layout": layout}


def conv_to_torch(inputs: dict, device, io_dtype: str = "f32") -> dict:
    """Move a conv problem to ``device``: x and the window in ``io_dtype`` (round to
    nearest even for bf16), weight and bias float32; x keeps its storage layout."""
    import torch

    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[io_dtype]
    x = inputs["x"]
    if inputs["layout"] == "bld":
        t = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1)))
        t = t.to(device=device, dtype=dt).transpose(1, 2)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dt)
    return {
        "x": t,
        "weight": torch.from_numpy(inputs["weight"]).to(device),
        "bias": torch.from_numpy(inputs["bias"]).to(device),
        "window": torch.from_numpy(inputs["window"]).to(device=device, dtype=dt),
        "layout": inputs["layout"],
    }


def conv_algorithmic_bytes(batch: int, dim: int, seqlen: int, width: int, io_bytes: int,
                           has_bias: bool = True) -> int:
    """Bytes the conv1d must move: x read once, out written once, taps and bias."""
    return 2 * batch * dim * seqlen * io_bytes + dim * width * 4 + (dim * 4 if has_bias else 0)
