"""GPU parity of the selective-scan backward against the fp64 backward oracle.

Tolerances (error metric: max |o - r| / (|r| + rms(r)), per gradient tensor):
  fp32 I/O 1e-4, as for the forward: every gradient is a short fp32 sum
      (over the 16 states, the 8 channels of a wave and then the 64 of a
      workgroup, or the steps of one channel) of products of quantities that
      the forward's own 1e-4 already bounds, and the reverse adjoint g obeys
      the same contracting recurrence as the forward state;
  bf16 I/O 2e-2: the oracle reads the same rounded inputs; the gradients that
      are stored in bf16 carry a rounding of at most 2^-9 on top of the fp32
      error, and the fp32 ones (dA_log, dD, ddt_bias, dinitial_state) inherit
      the bf16 rounding of nothing but their inputs.
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, device, note, to_np
from mamba_selective_scan_amd.inputs import WORKLOADS, generate

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
ORACLE_NAME = {"du": "du", "ddelta_raw": "ddelta_raw", "dA_log": "dA_log", "dB": "dB",
               "dC": "dC", "dD": "dD", "dz": "dz", "ddt_bias": "ddt_bias",
               "dinitial_state": "dh0"}


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _problem(batch, dim, seqlen, dstate, layout="bdl", io="f32", seed=0, softplus=True,
             with_z=True, with_D=True, with_bias=True, h0=False, dfinal=False,
             a_log="ladder"):
    import torch
    from mamba_selective_scan_amd.inputs import to_torch
    x = generate(batch, dim, seqlen, dstate, layout, seed=seed, a_log=a_log)
    if not softplus:
        x["dt_bias"] = np.log1p(np.exp(x["dt_bias"].astype(np.float64))).astype(np.float32)
        x["delta_raw"] = np.abs(x["delta_raw"]) * np.float32(0.1)
    dx = to_torch(x, device(), io)
    g = torch.Generator().manual_seed(seed + 7)
    dt = dx["u"].dtype
    dout = torch.randn(batch, dim, seqlen, generator=g)
    if layout == "bld":
        dout = dout.transpose(1, 2).contiguous().transpose(1, 2)
    dx["dout"] = dout.to(device=device(), dtype=dt)
    dx["h0"] = torch.randn(batch, dim, dstate, generator=g).to(device()) if h0 else None
    dx["dfinal"] = torch.randn(batch, dim, dstate, generator=g).to(device()) if dfinal else None
    if not with_z:
        dx["z"] = None
    if not with_D:
        dx["D"] = None
    if not with_bias:
        dx["dt_bias"] = None
    return dx


def _run_and_check(mss, name, dx, io="f32", softplus=True):
    import torch
    note(f"bwd {name}: shape={tuple(dx['u'].shape)} N={dx['A_log'].shape[1]} {io} "
         f"softplus={softplus} z={dx['z'] is not None} D={dx['D'] is not None} "
         f"bias={dx['dt_bias'] is not None} h0={dx['h0'] is not None} "
         f"dfinal={dx['dfinal'] is not None}")
    got = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                 dx["dout"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                 delta_softplus=softplus, initial_state=dx["h0"],
                                 dfinal_state=dx["dfinal"])
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dx["dout"],
                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], h0=dx["h0"],
                          dfinal=dx["dfinal"], delta_softplus=softplus)
    for k, v in got.items():
        check(f"bwd {name} {k}", to_np(v), ref[ORACLE_NAME[k]], TOL[io])
    expect = {"du", "ddelta_raw", "dA_log", "dB", "dC"}
    expect |= {"dD"} if dx["D"] is not None else set()
    expect |= {"dz"} if dx["z"] is not None else set()
    expect |= {"ddt_bias"} if dx["dt_bias"] is not None else set()
    expect |= {"dinitial_state"} if dx["h0"] is not None else set()
    assert set(got) == expect
    return got


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_workload(mss, seed):
    w = WORKLOADS["tiny"]
    _run_and_check(mss, "tiny", _problem(w.batch, w.dim, w.seqlen, w.dstate, seed=seed,
                                         h0=True, dfinal=True))


def test_mamba130m_layer(mss):
    w = WORKLOADS["mamba130m_layer"]
    _run_and_check(mss, "130m", _problem(w.batch, w.dim, w.seqlen, w.dstate))


@pytest.mark.parametrize("seqlen", [1, 7, 16, 17, 33, 100])
def test_ragged_lengths(mss, seqlen):
    _run_and_check(mss, f"L={seqlen}", _problem(2, 72, seqlen, 16, h0=True, dfinal=True))


@pytest.mark.parametrize("dstate", [1, 5, 13])
def test_small_dstate(mss, dstate):
    _run_and_check(mss, f"N={dstate}", _problem(2, 130, 90, dstate))


@pytest.mark.parametrize("flags", [dict(with_z=False), dict(with_D=False), dict(with_bias=False),
                                   dict(softplus=False), dict(h0=True),
                                   dict(with_z=False, with_D=False, h0=True, dfinal=True)])
def test_optional_inputs(mss, flags):
    softplus = flags.get("softplus", True)
    _run_and_check(mss, f"{flags}", _problem(2, 96, 150, 16, **flags), softplus=softplus)


@pytest.mark.parametrize("shape", [(1, 64, 2000), (1, 200, 1500), (3, 40, 999)])
def test_time_segments(mss, shape):
    # few channels and long sequences: the backward splits time into segments
    # joined by forward state carries and backward adjoint carries
    batch, dim, seqlen = shape
    _run_and_check(mss, f"segments {shape}", _problem(batch, dim, seqlen, 16, h0=True,
                                                      dfinal=True, a_log="normal"))


def test_long_sequence(mss):
    """The 32k-token sequence length at 384 channels (a time-split backward with
    many segments): every gradient against the oracle, element by element."""
    import torch
    w = WORKLOADS["long_handoff"]
    dx = _problem(w.batch, 384, w.seqlen, w.dstate, dfinal=True)
    note(f"bwd long shape: B={w.batch} D=384 L={w.seqlen}")
    got = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                 dx["dout"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                 dfinal_state=dx["dfinal"])
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dx["dout"],
                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], dfinal=dx["dfinal"])
    for k, v in got.items():
        check(f"bwd long {k}", to_np(v), ref[ORACLE_NAME[k]], TOL["f32"])


def _oracle_bwd_in_channel_groups(dx, groups=8):
    """The oracle backward over every channel, run on channel groups in
    threads (the oracle's C call releases the GIL).  Channels are independent
    except through dB and dC, which sum over them: the groups' dB and dC are
    added (in fp64), every other gradient comes from its channel's group."""
    from concurrent.futures import ThreadPoolExecutor
    oracle.load()
    host = {k: (None if dx.get(k) is None else to_np(dx[k]))
            for k in ("u", "delta_raw", "A_log", "B", "C", "dout", "D", "z", "dt_bias", "h0",
                      "dfinal")}
    dim = host["u"].shape[1]
    edges = np.linspace(0, dim, groups + 1).astype(int)

    def run(i):
        c = slice(edges[i], edges[i + 1])
        opt = lambda k, ax: None if host[k] is None else (host[k][:, c] if ax else host[k][c])  # noqa: E731
        return oracle.scan_bwd(host["u"][:, c], host["delta_raw"][:, c], host["A_log"][c],
                               host["B"], host["C"], host["dout"][:, c], D=opt("D", 0),
                               z=opt("z", 1), dt_bias=opt("dt_bias", 0), h0=opt("h0", 1),
                               dfinal=opt("dfinal", 1))

    with ThreadPoolExecutor(groups) as pool:
        parts = list(pool.map(run, range(groups)))
    ref = {}
    for k in parts[0]:
        if parts[0][k] is None:
            ref[k] = None
        elif k in ("dB", "dC"):
            ref[k] = sum(p[k] for p in parts)
        else:
            ref[k] = np.concatenate([p[k] for p in parts], axis=0 if k in ("dA_log", "dD",
                                                                           "ddt_bias") else 1)
    return ref


@pytest.mark.parametrize("wname", ["mamba130m_layer", "long_handoff", "audio_channel_last"])
def test_few_channel_workloads_full(mss, wname):
    """The few-channel workloads at their full shapes, in the launch
    configuration bench.py times (time segments; the aggregate pass in parts
    when the forward's chunk states are given; channel-last rows on the audio
    shape), with initial state and final-state gradient: the standalone
    backward and the backward reading the forward's chunk states, every
    gradient of every channel against the oracle."""
    import torch
    w = WORKLOADS[wname]
    dx = _problem(w.batch, w.dim, w.seqlen, w.dstate, layout=w.layout, h0=True, dfinal=True)
    note(f"bwd full {wname}: B={w.batch} D={w.dim} L={w.seqlen} {w.layout}")
    args = (dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dx["dout"])
    kw = dict(D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=dx["h0"],
              dfinal_state=dx["dfinal"])
    standalone = mss.selective_scan_bwd(*args, **kw)
    _, states = mss.selective_scan_fwd(*args[:5], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                       initial_state=dx["h0"], return_chunk_states=True)
    with_states = mss.selective_scan_bwd(*args, **kw, chunk_states=states)
    torch.cuda.synchronize()
    ref = _oracle_bwd_in_channel_groups(dx)
    for name, got in (("standalone", standalone), ("with chunk states", with_states)):
        for k, v in got.items():
            check(f"bwd full {wname} {name} {k}", to_np(v), ref[ORACLE_NAME[k]], TOL["f32"])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_mamba2p8b_layer_full(mss, io):
    """The 2.8b layer shape (8 x 5120 x 4096) in the launch configuration
    bench.py times, with initial state and final-state gradient: one whole
    batch row against the oracle run on that row (every gradient of the row,
    dB and dC included, since they sum over the row's channels), and a channel
    sample across all rows for the gradients that sum over rows (dA_log, dD,
    ddt_bias)."""
    import torch
    w = WORKLOADS["mamba2p8b_layer"]
    dx = _problem(w.batch, w.dim, w.seqlen, w.dstate, io=io, h0=True, dfinal=True)
    note(f"bwd full 2.8b layer {io}")
    got = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                 dx["dout"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                 initial_state=dx["h0"], dfinal_state=dx["dfinal"])
    torch.cuda.synchronize()
    tol = TOL[io]
    b = 5
    rows = {k: dx[k][b:b + 1] for k in ("u", "delta_raw", "B", "C", "dout", "z", "h0", "dfinal")}
    ref = oracle.scan_bwd(rows["u"], rows["delta_raw"], dx["A_log"], rows["B"], rows["C"],
                          rows["dout"], D=dx["D"], z=rows["z"], dt_bias=dx["dt_bias"],
                          h0=rows["h0"], dfinal=rows["dfinal"])
    for k in ("du", "ddelta_raw", "dz", "dB", "dC", "dinitial_state"):
        check(f"bwd full {io} row {b} {k}", to_np(got[k][b:b + 1]), ref[ORACLE_NAME[k]], tol)
    rng = np.random.default_rng(17)
    chans = np.unique(np.concatenate([[0, 31, 32, w.dim - 1], rng.choice(w.dim, 20, replace=False)]))
    ci = torch.as_tensor(chans, device=device())
    sub = {k: dx[k][:, ci] for k in ("u", "delta_raw", "dout", "z", "h0", "dfinal")}
    ref2 = oracle.scan_bwd(sub["u"], sub["delta_raw"], dx["A_log"][ci], dx["B"], dx["C"],
                           sub["dout"], D=dx["D"][ci], z=sub["z"], dt_bias=dx["dt_bias"][ci],
                           h0=sub["h0"], dfinal=sub["dfinal"])
    for k in ("dA_log", "dD", "ddt_bias"):
        check(f"bwd full {io} sampled {k}", to_np(got[k][ci]), ref2[ORACLE_NAME[k]], tol)
    for k in ("du", "ddelta_raw", "dz", "dinitial_state"):
        check(f"bwd full {io} sampled {k}", to_np(got[k][:, ci]), ref2[ORACLE_NAME[k]], tol)
    # the same backward reading the forward's chunk states
    _, states = mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                       D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                       initial_state=dx["h0"], return_chunk_states=True)
    got2 = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                  dx["dout"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                  initial_state=dx["h0"], dfinal_state=dx["dfinal"],
                                  chunk_states=states)
    torch.cuda.synchronize()
    for k in ("du", "dB", "dA_log", "dinitial_state"):
        check(f"bwd full {io} with chunk states {k}", to_np(got2[k][b:b + 1] if k != "dA_log"
                                                            else got2[k]),
              to_np(got[k][b:b + 1] if k != "dA_log" else got[k]), 1e-5 if io == "f32" else 1e-2)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("big_bias", [False, True])
def test_softplus_upper_range(mss, io, big_bias):
    """delta_raw + dt_bias over [-40, 40] (a dense grid through 19.5..20.5,
    values above 30; dt_bias 0 or 25): softplus and its derivative sigmoid in
    the backward against the oracle, every gradient element by element."""
    from mamba_selective_scan_amd.inputs import softplus_range_delta
    dx = _problem(2, 72, 300, 16, io=io, h0=True, dfinal=True)
    dr, bias = softplus_range_delta(2, 72, 300, seed=3, big_bias=big_bias)
    import torch
    dx["delta_raw"] = torch.from_numpy(dr).to(device=device(), dtype=dx["u"].dtype)
    dx["dt_bias"] = torch.from_numpy(bias).to(device())
    _run_and_check(mss, f"softplus range {io} big_bias={big_bias}", dx, io=io)


def test_time_invariant_B_C(mss):
    """B and C constant in time, passed as stride-0 views: the gradient of the
    [B, N] parameters is the time sum of dB and dC."""
    import torch
    dx = _problem(2, 96, 300, 16, h0=True)
    g = torch.Generator().manual_seed(4)
    base = {k: torch.randn(2, 16, generator=g).to(device()) for k in ("B", "C")}
    for k in ("B", "C"):
        dx[k] = base[k][:, :, None].expand(2, 16, 300)
    got = _run_and_check(mss, "time-invariant B/C", dx)
    ref = oracle.scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dx["dout"],
                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], h0=dx["h0"])
    for k, r in (("dB", "dB"), ("dC", "dC")):
        check(f"bwd time-invariant sum_t {k}", to_np(got[k]).sum(axis=2), ref[r].sum(axis=2),
              TOL["f32"])


def test_random_a_log(mss):
    _run_and_check(mss, "A_log~N(0,1)", _problem(1, 128, 300, 16, a_log="normal", h0=True))


def test_channel_last_layout(mss):
    _run_and_check(mss, "bld", _problem(2, 64, 200, 16, layout="bld", h0=True, dfinal=True))


@pytest.mark.parametrize("case", [
    (1, 50, 3000, "f32"),   # time segments, a partly empty 32-channel block
    (2, 40, 333, "bf16"),   # bf16, partly empty block, ragged chunk
    (8, 3072, 48, "f32"),   # 768 (row, block) pairs: no time segments
])
def test_channel_last_cooperative_rows(mss, case):
    """Channel-last inputs: with time segments, the aggregate and checkpoint
    passes' workgroups load whole 128-byte rows of their 32-channel tiles and
    stage them in LDS for the waves that walk them."""
    batch, dim, seqlen, io = case
    _run_and_check(mss, f"bld coop {case}",
                   _problem(batch, dim, seqlen, 16, layout="bld", io=io, h0=True, dfinal=True),
                   io=io)


@pytest.mark.parametrize("batch,dim,seqlen,io,with_z", [
    (2, 96, 130, "f32", False),   # no z: no dz rows to store
    (3, 34, 45, "bf16", True),    # a 2-channel last tile, odd batch, ragged chunk
])
def test_channel_last_gradient_rows(mss, batch, dim, seqlen, io, with_z):
    """Channel-last inputs and gradients without z (no dz rows), and with a last
    32-channel tile that holds 2 channels, an odd batch and a ragged chunk."""
    _run_and_check(mss, f"bld rows B={batch} D={dim} L={seqlen} {io} z={with_z}",
                   _problem(batch, dim, seqlen, 16, layout="bld", io=io, with_z=with_z,
                            h0=True, dfinal=True),
                   io=io)


@pytest.mark.parametrize("dstate,io,states,dim", [(5, "f32", False, 80), (3, "f32", True, 80),
                                                   (16, "bf16", True, 80), (8, "bf16", False, 80),
                                                   (16, "f32", False, 77), (16, "f32", True, 77)])
def test_channel_last_segments_small_dstate_and_states(mss, dstate, io, states, dim):
    """Channel-last, time segments (1 x 80 x 1900: 3 tiles, the last half
    empty, 14 segments), with dstate below 16 (B, C element by element when it
    is not a multiple of 4, 4-state vectors when it is; dB and dC summed with
    lanes past dstate idle) and with or without the forward's chunk states
    (the aggregate pass without H).  An odd channel count (77) cannot move
    channel pairs: the one-wave aggregate and checkpoint passes with element
    loads."""
    import torch
    dx = _problem(1, dim, 1900, dstate, layout="bld", io=io, h0=True, dfinal=True)
    kw = {}
    if states:
        _, kw["chunk_states"] = mss.selective_scan_fwd(
            dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], D=dx["D"], z=dx["z"],
            dt_bias=dx["dt_bias"], initial_state=dx["h0"], return_chunk_states=True)
    note(f"bwd bld segments D={dim} N={dstate} {io} states={states}")
    got = mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                 dx["dout"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                 initial_state=dx["h0"], dfinal_state=dx["dfinal"], **kw)
    torch.cuda.synchronize()
    ref = oracle.scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dx["dout"],
                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], h0=dx["h0"],
                          dfinal=dx["dfinal"])
    for k, v in got.items():
        check(f"bwd bld segments D={dim} N={dstate} {io} states={states} {k}", to_np(v),
              ref[ORACLE_NAME[k]], TOL[io])


@pytest.mark.parametrize("seqlen", [200, 201])
def test_bf16(mss, seqlen):
    # an even length moves the step pairs as one 32-bit access; an odd one
    # takes the element-wise path
    _run_and_check(mss, f"bf16 L={seqlen}",
                   _problem(2, 128, seqlen, 16, io="bf16", h0=True, dfinal=True), io="bf16")


def _relayout(t, unit_axis):
    """The same logical [B, X, L] values stored with unit stride on axis 1
    (channels or states) or axis 2 (time)."""
    if unit_axis == 2:
        return t.contiguous()
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("x_axis,bc_axis", [(2, 1), (1, 2)])
def test_mixed_layouts(mss, x_axis, bc_axis):
    """u, delta_raw, z, dout in one layout and B, C in the other: the
    checkpoint pass reads u, delta_raw as 4-step vectors but B element-wise,
    or the reverse; dB and dC keep the layout of B and C."""
    dx = _problem(2, 72, 256, 16, h0=True, dfinal=True)
    for k in ("u", "delta_raw", "z", "dout"):
        dx[k] = _relayout(dx[k], x_axis)
    for k in ("B", "C"):
        dx[k] = _relayout(dx[k], bc_axis)
    _run_and_check(mss, f"x axis {x_axis}, B/C axis {bc_axis}", dx)


def test_B_odd_row_pitch(mss):
    """B and C as views with rows of odd pitch: B element-wise in the
    checkpoint pass while u, delta_raw stay vectors."""
    import torch
    dx = _problem(2, 64, 128, 16, h0=True, dfinal=True)
    for k in ("B", "C"):
        wide = torch.zeros(2, 16, 129, device=device(), dtype=dx[k].dtype)
        wide[:, :, :128] = dx[k]
        dx[k] = wide[:, :, :128]
    assert dx["B"].stride(1) == 129
    _run_and_check(mss, "B odd row pitch", dx)


def test_odd_row_stride(mss):
    """Even length but rows of odd pitch (views into a wider buffer): the
    element-wise path, since a step pair would straddle an 8-byte boundary."""
    import torch
    dx = _problem(2, 96, 120, 16, h0=True, dfinal=True)
    for k in ("u", "delta_raw", "z", "dout"):
        wide = torch.zeros(2, 96, 121, device=device(), dtype=dx[k].dtype)
        wide[:, :, :120] = dx[k]
        dx[k] = wide[:, :, :120]
    assert dx["u"].stride(1) == 121
    _run_and_check(mss, "odd row stride", dx)


def test_run_twice_bitwise(mss):
    import torch
    dx = _problem(2, 130, 77, 16, h0=True, dfinal=True)
    note("bwd run-twice determinism")
    args = (dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dx["dout"])
    kw = dict(D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=dx["h0"],
              dfinal_state=dx["dfinal"])
    a = mss.selective_scan_bwd(*args, **kw)
    b = mss.selective_scan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("reverse", [False, True])
def test_autograd_function(mss, reverse):
    """selective_scan under torch.autograd: loss = sum(w * out) + sum(v * final)
    gives the oracle's gradients for dout = w, dfinal = v."""
    import torch
    dx = _problem(2, 64, 120, 16, h0=True)
    g = torch.Generator().manual_seed(9)
    w = torch.randn(2, 64, 120, generator=g).to(device())
    v = torch.randn(2, 64, 16, generator=g).to(device())
    names = ["u", "delta_raw", "A_log", "B", "C", "D", "z", "dt_bias", "h0"]
    leaves = {k: dx[k].detach().clone().requires_grad_(True) for k in names}
    note(f"autograd function reverse={reverse}")
    out, fin = mss.selective_scan(leaves["u"], leaves["delta_raw"], leaves["A_log"],
                                  leaves["B"], leaves["C"], leaves["D"], leaves["z"],
                                  leaves["dt_bias"], initial_state=leaves["h0"],
                                  reverse=reverse, return_final_state=True)
    ((out * w).sum() + (fin * v).sum()).backward()
    torch.cuda.synchronize()
    flip = (lambda a: np.ascontiguousarray(to_np(a)[:, :, ::-1])) if reverse else to_np
    ref = oracle.scan_bwd(flip(dx["u"]), flip(dx["delta_raw"]), dx["A_log"], flip(dx["B"]),
                          flip(dx["C"]), flip(w), D=dx["D"], z=flip(dx["z"]),
                          dt_bias=dx["dt_bias"], h0=dx["h0"], dfinal=v)
    oname = {"u": "du", "delta_raw": "ddelta_raw", "A_log": "dA_log", "B": "dB", "C": "dC",
             "D": "dD", "z": "dz", "dt_bias": "ddt_bias", "h0": "dh0"}
    for k in names:
        r = ref[oname[k]]
        if reverse and k in ("u", "delta_raw", "B", "C", "z"):
            r = r[:, :, ::-1]
        check(f"autograd grad {k} reverse={reverse}", to_np(leaves[k].grad), r, TOL["f32"])


@pytest.mark.parametrize("loss", ["out.sum", "fin.sum", "both.mean", "out.sum bf16"])
def test_autograd_reduction_losses(mss, loss):
    """Losses built from sum() and mean(): their gradients reach the backward
    as expanded stride-0 views (dout from out.sum(), dfinal from fin.sum()),
    and give the oracle's gradients for a constant dout and dfinal."""
    import torch
    io = "bf16" if loss.endswith("bf16") else "f32"
    dx = _problem(2, 64, 120, 16, io=io, h0=True)
    names = ["u", "delta_raw", "A_log", "B", "C", "D", "z", "dt_bias", "h0"]
    leaves = {k: dx[k].detach().clone().requires_grad_(True) for k in names}
    note(f"autograd {loss}")
    out, fin = mss.selective_scan(leaves["u"], leaves["delta_raw"], leaves["A_log"],
                                  leaves["B"], leaves["C"], leaves["D"], leaves["z"],
                                  leaves["dt_bias"], initial_state=leaves["h0"],
                                  return_final_state=True)
    n_out, n_fin = out.numel(), fin.numel()
    if loss.startswith("out.sum"):
        out.sum().backward()
        w, v = 1.0, 0.0
    elif loss == "fin.sum":
        fin.sum().backward()
        w, v = 0.0, 1.0
    else:
        (out.mean() + fin.mean()).backward()
        w, v = 1.0 / n_out, 1.0 / n_fin
    torch.cuda.synchronize()
    dout = np.full(tuple(out.shape), w)
    dfin = np.full(tuple(fin.shape), v)
    ref = oracle.scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], dout,
                          D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], h0=dx["h0"], dfinal=dfin)
    oname = {"u": "du", "delta_raw": "ddelta_raw", "A_log": "dA_log", "B": "dB", "C": "dC",
             "D": "dD", "z": "dz", "dt_bias": "ddt_bias", "h0": "dh0"}
    for k in names:
        check(f"autograd {loss} grad {k}", to_np(leaves[k].grad), ref[oname[k]], TOL[io])
