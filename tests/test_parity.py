"""GPU parity: the HIP path against the fp64 oracle on seeded synthetic inputs.

Tolerances (error metric: max |o - r| / (|r| + rms(r))): 1e-4 for fp32 I/O,
2e-2 for bf16 I/O with fp32 state.  Small problems are compared element by
element everywhere; full-size workloads are compared on sampled channels, each
over its whole sequence (the oracle computes one channel at a time), plus the
exported final state of those channels.
"""

import numpy as np
import pytest

import oracle
from gpu_util import (check, device, note, oracle_full, run_gpu, sample_channels, to_np,
                      tol_for)
from mamba_selective_scan_amd.inputs import WORKLOADS, generate, generate_workload, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _full_case(mss, name, batch, dim, seqlen, dstate, layout="bdl", io="f32", seed=0,
               a_log="ladder", d_skip="ones", **flags):
    note(f"{name}: B={batch} D={dim} L={seqlen} N={dstate} {layout} {io} seed={seed} {flags}")
    x = generate(batch, dim, seqlen, dstate, layout, seed=seed, a_log=a_log, d_skip=d_skip)
    if not flags.get("softplus", True):
        # Without softplus delta = delta_raw + dt_bias is used as is; keep it
        # positive (dt_bias = the time step itself, |delta_raw| scaled down) so
        # the recurrence stays bounded (a negative delta makes |a| > 1).
        x["dt_bias"] = np.log1p(np.exp(x["dt_bias"].astype(np.float64))).astype(np.float32)
        x["delta_raw"] = np.abs(x["delta_raw"]) * np.float32(0.1)
    dx = to_torch(x, device(), io)
    h0 = flags.pop("h0", False)
    init = None
    if h0:
        import torch
        g = torch.Generator().manual_seed(seed + 100)
        init = torch.randn(batch, dim, dstate, generator=g).to(device())
    out, fin = run_gpu(mss, dx, initial_state=init, **flags)
    import torch
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle_full(dx, initial_state=init, **flags)
    tol = tol_for(io)
    check(f"{name} out", to_np(out), ref_out, tol)
    check(f"{name} final_state", to_np(fin), ref_fin, tol)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_workload(mss, seed):
    w = WORKLOADS["tiny"]
    _full_case(mss, "tiny", w.batch, w.dim, w.seqlen, w.dstate, seed=seed)


def test_mamba130m_layer_full(mss):
    w = WORKLOADS["mamba130m_layer"]
    _full_case(mss, "mamba130m_layer", w.batch, w.dim, w.seqlen, w.dstate)


@pytest.mark.parametrize("seqlen", [1, 7, 31, 33, 63, 2049, 4097])
def test_ragged_lengths(mss, seqlen):
    _full_case(mss, f"ragged L={seqlen}", 2, 72, seqlen, 16)


@pytest.mark.parametrize("dstate", [1, 3, 4, 5, 13])
def test_small_dstate(mss, dstate):
    _full_case(mss, f"dstate={dstate}", 1, 130, 300, dstate)


@pytest.mark.parametrize("flags", [
    dict(with_z=False), dict(with_D=False), dict(with_bias=False), dict(softplus=False),
    dict(with_z=False, with_D=False), dict(h0=True), dict(with_z=False, with_D=False, h0=True),
])
def test_optional_inputs(mss, flags):
    _full_case(mss, f"flags {sorted(flags)}", 2, 100, 777, 16, **dict(flags))


def test_random_A_log_and_D(mss):
    _full_case(mss, "random A_log, D", 2, 128, 1000, 16, a_log="normal", d_skip="normal")


def test_ssm_only_term(mss):
    """D = 0 and no gate: the output is the scan term alone."""
    _full_case(mss, "ssm only", 1, 192, 2048, 16, d_skip="zeros", with_z=False, with_D=False)


@pytest.mark.parametrize("seqlen", [100, 5000])
def test_channel_last_layout_small(mss, seqlen):
    _full_case(mss, f"bld L={seqlen}", 1, 100, seqlen, 16, layout="bld")


@pytest.mark.parametrize("seqlen", [70, 3000])
def test_bf16_small(mss, seqlen):
    _full_case(mss, f"bf16 L={seqlen}", 2, 96, seqlen, 16, io="bf16")


@pytest.mark.parametrize("layout,dim,seqlen", [("bdl", 1536, 2048), ("bld", 256, 3000),
                                               ("bld", 200, 1001), ("bdl", 64, 4099)])
def test_bf16_batch_one(mss, layout, dim, seqlen):
    """bf16 at batch 1 (the size-1 batch stride is never stepped, so it does
    not keep the vector paths out), channel-last with time segments and a
    channel count that is not a whole 32-channel block, and a ragged tail."""
    _full_case(mss, f"bf16 B=1 {layout}", 1, dim, seqlen, 16, layout=layout, io="bf16", h0=True)


def test_time_split_with_initial_state(mss):
    """Few channels and a long sequence: the segmented path, started from h0."""
    _full_case(mss, "split+h0", 1, 64, 20000, 16, h0=True)


@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_aggregate_pass_in_parts(mss, layout):
    """1x8192x1117: four time segments of 9 chunks (the last one ragged), the
    aggregate pass cut into parts of 5 and 4 chunks (8192 channels in four
    segments fill only half of its eight waves per SIMD), started from h0,
    with a ragged tail; both layouts against the oracle."""
    _full_case(mss, f"aggregate parts {layout}", 1, 8192, 1117, 16, layout=layout, h0=True)


@pytest.mark.parametrize("shared_batch", [False, True])
@pytest.mark.parametrize("seqlen", [77, 4096])
def test_time_invariant_B_C(mss, shared_batch, seqlen):
    """Time-invariant B and C (the S4-style variant): [B, N] (or [N]) tensors
    broadcast along time as stride-0 views, with no copy."""
    import torch
    bsz, dim, N = 2, 96, 16
    note(f"time-invariant B/C L={seqlen} shared_batch={shared_batch}")
    x = generate(bsz, dim, seqlen, N, seed=11)
    dx = to_torch(x, device(), "f32")
    g = torch.Generator().manual_seed(3)
    for k in ("B", "C"):
        if shared_batch:
            base = torch.randn(N, generator=g).to(device())
            dx[k] = base[None, :, None].expand(bsz, N, seqlen)
        else:
            base = torch.randn(bsz, N, generator=g).to(device())
            dx[k] = base[:, :, None].expand(bsz, N, seqlen)
        assert dx[k].stride()[2] == 0
    out, fin = run_gpu(mss, dx)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle_full(dx)
    check(f"time-invariant B/C L={seqlen} out", to_np(out), ref_out, 1e-4)
    check(f"time-invariant B/C L={seqlen} final", to_np(fin), ref_fin, 1e-4)


def _lti_inputs(batch, dim, seqlen, dstate, layout, io, seed, source="expand"):
    """A workload with B and C replaced by [batch, dstate] values broadcast
    along time (stride-0 views): of a [batch, dstate] tensor ("expand", state
    stride 1) or of the workload's own first step ("slice", the state stride of
    its layout: seqlen for [B,N,L])."""
    import torch
    x = generate(batch, dim, seqlen, dstate, layout, seed=seed)
    dx = to_torch(x, device(), io)
    g = torch.Generator().manual_seed(seed + 5)
    for k in ("B", "C"):
        if source == "slice":
            dx[k] = dx[k][:, :, :1].expand(batch, dstate, seqlen)
        else:
            base = torch.randn(batch, dstate, generator=g).to(device(), dx["u"].dtype)
            dx[k] = base[:, :, None].expand(batch, dstate, seqlen)
    return dx


def _materialised(t, layout):
    """The same values with a real time axis, in the workload's B/C layout."""
    if layout == "bld":
        return t.transpose(1, 2).contiguous().transpose(1, 2)
    return t.contiguous()


@pytest.mark.parametrize("source", ["expand", "slice"])
@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_time_invariant_register_path_equals_materialised(mss, layout, io, reverse, source):
    """Time-invariant B/C take the vector pass that holds B and C in registers;
    the same values materialised along time take the path through LDS.  Both
    do the same arithmetic in the same order, so the results are bitwise equal.
    The length leaves a ragged tail for the element-wise pass."""
    import torch
    batch, dim, seqlen, N = 2, 96, 1002, 16
    note(f"LTI vs materialised: {layout} {io} reverse={reverse} L={seqlen} {source}")
    dx = _lti_inputs(batch, dim, seqlen, N, layout, io, seed=21, source=source)
    dm = dict(dx)
    for k in ("B", "C"):
        dm[k] = _materialised(dx[k], layout)
        assert dx[k].stride()[2] == 0 and dm[k].stride()[2] != 0
    res = []
    for d_in in (dx, dm):
        res.append(mss.selective_scan_fwd(
            d_in["u"], d_in["delta_raw"], d_in["A_log"], d_in["B"], d_in["C"], D=d_in["D"],
            z=d_in["z"], dt_bias=d_in["dt_bias"], reverse=reverse, return_final_state=True,
            return_chunk_states=True))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]), "outputs differ"
    assert torch.equal(res[0][1], res[1][1]), "final states differ"
    assert torch.equal(res[0][2], res[1][2]), "chunk states differ"
    if not reverse:
        ref_out, ref_fin = oracle_full(dx)
        check(f"LTI {layout} {io} out", to_np(res[0][0]), ref_out, tol_for(io))
        check(f"LTI {layout} {io} final", to_np(res[0][1]), ref_fin, tol_for(io))


@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_time_invariant_split_h0_odd_dstate(mss, layout):
    """Few channels and a long sequence with time-invariant B/C: aggregate
    pass, carries and main pass all hold B and C in registers, from an initial
    state.  dstate 5 is not a whole number of 4-element vectors, which the
    register path does not need."""
    import torch
    batch, dim, seqlen, N = 1, 64, 20000, 5
    note(f"LTI split+h0 {layout} B={batch} D={dim} L={seqlen} N={N}")
    dx = _lti_inputs(batch, dim, seqlen, N, layout, "f32", seed=33)
    g = torch.Generator().manual_seed(34)
    init = torch.randn(batch, dim, N, generator=g).to(device())
    out, fin = run_gpu(mss, dx, initial_state=init)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle_full(dx, initial_state=init)
    check(f"LTI split {layout} out", to_np(out), ref_out, 1e-4)
    check(f"LTI split {layout} final", to_np(fin), ref_fin, 1e-4)


@pytest.mark.parametrize("layout", ["bdl", "bld"])
def test_views_into_padded_buffers(mss, layout):
    """Views with offsets and padded row strides (the unit-stride axis kept)."""
    import torch
    note(f"padded views {layout}")
    bsz, dim, L, N = 2, 80, 301, 16
    x = generate(bsz, dim, L, N, seed=5)
    dx = to_torch(x, device(), "f32")
    big = {}
    for k in ("u", "delta_raw", "z"):
        if layout == "bdl":
            buf = torch.zeros(bsz, dim + 9, L + 11, device=device())
            buf[:, 1:1 + dim, 5:5 + L] = dx[k]
            big[k] = buf[:, 1:1 + dim, 5:5 + L]
        else:
            buf = torch.zeros(bsz, L + 11, dim + 9, device=device())
            buf[:, 5:5 + L, 1:1 + dim] = dx[k].transpose(1, 2)
            big[k] = buf[:, 5:5 + L, 1:1 + dim].transpose(1, 2)
    for k in ("B", "C"):
        if layout == "bdl":
            buf = torch.zeros(bsz, N + 3, L + 7, device=device())
            buf[:, 2:2 + N, 3:3 + L] = dx[k]
            big[k] = buf[:, 2:2 + N, 3:3 + L]
        else:
            buf = torch.zeros(bsz, L + 7, N + 3, device=device())
            buf[:, 3:3 + L, 2:2 + N] = dx[k].transpose(1, 2)
            big[k] = buf[:, 3:3 + L, 2:2 + N].transpose(1, 2)
    for k in ("A_log", "D", "dt_bias"):
        big[k] = dx[k]
    out, fin = run_gpu(mss, big)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle_full(dx)
    check(f"padded views {layout} out", to_np(out), ref_out, 1e-4)
    check(f"padded views {layout} final", to_np(fin), ref_fin, 1e-4)


def _run_pair(mss, a, b):
    """Run the forward on two argument dicts; both results, synchronised."""
    import torch
    ra = mss.selective_scan_fwd(a["u"], a["delta_raw"], a["A_log"], a["B"], a["C"], D=a["D"],
                                z=a["z"], dt_bias=a["dt_bias"], return_final_state=True)
    rb = mss.selective_scan_fwd(b["u"], b["delta_raw"], b["A_log"], b["B"], b["C"], D=b["D"],
                                z=b["z"], dt_bias=b["dt_bias"], return_final_state=True)
    torch.cuda.synchronize()
    return ra, rb


def _odd_pitch(t):
    """The same [B, X, L] values as a view into a buffer one step wider (the
    row pitch becomes odd)."""
    import torch
    wide = torch.zeros(t.shape[0], t.shape[1], t.shape[2] + 1, dtype=t.dtype, device=t.device)
    wide[:, :, :t.shape[2]] = t
    return wide[:, :, :t.shape[2]]


@pytest.mark.parametrize("case", ["bf16_odd_pitch", "channel_last_dim102", "nfast_bc_dstate5"])
def test_elementwise_equals_vector_path(mss, case):
    """Layouts whose 4-element vectors are not whole run the element-wise
    instantiation of the same kernel: the result is bit for bit the vector
    path's on the same values."""
    import torch
    note(f"element-wise vs vector path: {case}")
    if case == "bf16_odd_pitch":
        # bf16 rows of odd pitch: 8-byte vectors would not be 4-byte aligned
        dx = to_torch(generate(2, 96, 1000, 16, seed=31), device(), "bf16")
        ev = dict(dx)
        for k in ("u", "delta_raw", "z", "B", "C"):
            ev[k] = _odd_pitch(dx[k])
        assert ev["u"].stride(1) % 2 == 1
        (out_v, fin_v), (out_e, fin_e) = _run_pair(mss, dx, ev)
    elif case == "channel_last_dim102":
        # 104 channels take the vector path, 102 (not a whole number of
        # 4-channel vectors) the element-wise one; the first 102 channels must
        # agree (the same 13 channel tiles, the same time segments)
        big = to_torch(generate(1, 104, 3000, 16, "bld", seed=32), device(), "f32")
        small = {k: (v[:, :102] if k in ("u", "delta_raw", "z") else
                     v[:102] if k in ("A_log", "D", "dt_bias") else v) for k, v in big.items()}
        (out_v, fin_v), (out_e, fin_e) = _run_pair(mss, big, small)
        out_v, fin_v = out_v[:, :102], fin_v[:, :102]
    else:
        # dstate 5 with B, C stored [B, L, N] (n-fast, not whole vectors of
        # states) against the same values stored [B, N, L]
        dx = to_torch(generate(2, 80, 700, 5, seed=33), device(), "f32")
        nf = dict(dx)
        for k in ("B", "C"):
            nf[k] = dx[k].transpose(1, 2).contiguous().transpose(1, 2)
        assert nf["B"].stride(1) == 1
        (out_v, fin_v), (out_e, fin_e) = _run_pair(mss, dx, nf)
    assert torch.equal(out_v, out_e), "outputs differ"
    assert torch.equal(fin_v, fin_e), "final states differ"


def test_no_unit_stride_axis_is_rejected(mss):
    import torch
    from mamba_selective_scan_amd import MssError
    note("no unit-stride axis")
    dx = to_torch(generate(1, 16, 64, 16, seed=6), device(), "f32")
    buf = torch.zeros(1, 16, 128, device=device())
    strided = buf[:, :, ::2]
    with pytest.raises(MssError) as e:
        mss.selective_scan_fwd(strided, dx["delta_raw"], dx["A_log"], dx["B"], dx["C"])
    assert e.value.name == "MSS_ERR_BAD_STRIDE"


@pytest.mark.parametrize("layout", ["bdl", "bld"])
@pytest.mark.parametrize("big_bias", [False, True])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_softplus_upper_range(mss, io, big_bias, layout):
    """delta_raw + dt_bias swept over [-40, 40] (a dense grid through 19.5..20.5
    and values above 30), with dt_bias = 0 or 25: the kernel's softplus, which
    takes no threshold shortcut, against the oracle's exact one, element by
    element, with and without the gate and the skip term."""
    import torch
    from mamba_selective_scan_amd.inputs import softplus_range_delta
    bsz, dim, L, N = 2, 72, 600, 16
    for with_z, with_D in ((True, True), (False, False)):
        note(f"softplus upper range {io} big_bias={big_bias} {layout} z={with_z} D={with_D}")
        x = generate(bsz, dim, L, N, layout, seed=21, d_skip="ones" if with_D else "zeros")
        x["delta_raw"], x["dt_bias"] = softplus_range_delta(bsz, dim, L, seed=21,
                                                            big_bias=big_bias)
        dx = to_torch(x, device(), io)
        out, fin = run_gpu(mss, dx, with_z=with_z, with_D=with_D)
        torch.cuda.synchronize()
        ref_out, ref_fin = oracle_full(dx, with_z=with_z, with_D=with_D)
        tol = tol_for(io)
        tag = f"softplus range {io} bias={big_bias} {layout} z={with_z}"
        check(f"{tag} out", to_np(out), ref_out, tol)
        check(f"{tag} final_state", to_np(fin), ref_fin, tol)


# ------------------------------------------------------------ full workloads

def _sampled_workload(mss, wname, io, k, seed=0, whole_row=None):
    """The full workload on the GPU in the launch configuration bench.py
    times; the oracle on k sampled channels (whole sequences), and with
    ``whole_row`` on every channel of that batch row as well."""
    import torch
    w = WORKLOADS[wname]
    note(f"{wname} {io}: generating inputs")
    x = generate_workload(w, seed=seed)
    dx = to_torch(x, device(), io)
    note(f"{wname} {io}: GPU scan")
    out, fin = run_gpu(mss, dx)
    torch.cuda.synchronize()
    chans = sample_channels(w.batch, w.dim, k, seed)
    note(f"{wname} {io}: oracle on {len(chans)} channels")
    ref_out, ref_fin = oracle.scan_channels(dx, chans)
    got_out = np.stack([to_np(out[b, d]) for b, d in chans])
    got_fin = np.stack([to_np(fin[b, d]) for b, d in chans])
    tol = tol_for(io)
    check(f"{wname} {io} out (sampled)", got_out, ref_out, tol)
    check(f"{wname} {io} final (sampled)", got_fin, ref_fin, tol)
    if whole_row is not None:
        b = whole_row
        note(f"{wname} {io}: oracle on all {w.dim} channels of batch row {b}")
        row = [(b, d) for d in range(w.dim)]
        ref_out, ref_fin = oracle.scan_channels(dx, row)
        check(f"{wname} {io} out (row {b}, every channel)", to_np(out[b]), ref_out, tol)
        check(f"{wname} {io} final (row {b}, every channel)", to_np(fin[b]), ref_fin, tol)


def test_mamba2p8b_layer_fp32_sampled(mss):
    _sampled_workload(mss, "mamba2p8b_layer", "f32", 96, whole_row=5)


def test_mamba2p8b_layer_bf16_sampled(mss):
    _sampled_workload(mss, "mamba2p8b_layer", "bf16", 96, whole_row=3)


def test_audio_channel_last_sampled(mss):
    _sampled_workload(mss, "audio_channel_last", "f32", 48)


def test_golden_fixtures_on_gpu(mss):
    import golden_cases
    import torch
    for name in golden_cases.ALL:
        c = golden_cases.load(name)
        note(f"golden {name}")
        f32 = lambda a: torch.tensor(a, dtype=torch.float32, device=device())
        if c["kind"] == "conv":
            out, fin = mss.causal_conv1d_fwd(f32(c["x"]), f32(c["w"]), f32(c["bias"]),
                                             activation=None, return_final_state=True)
        elif c["kind"] == "conv_step":
            fin = f32(c["state"])
            out = mss.causal_conv1d_update(fin, f32(c["x"]), f32(c["w"]), f32(c["bias"]),
                                           activation=None)
        elif c["kind"] == "scan":
            out, fin = mss.selective_scan_fwd(f32(c["u"]), f32(c["delta_raw"]), f32(c["A_log"]),
                                              f32(c["B"]), f32(c["C"]), D=f32(c["D"]),
                                              delta_softplus=False, return_final_state=True)
        else:
            st = f32(c["state"])
            out = mss.selective_state_update(st, f32(c["u"]), f32(c["delta_raw"]), f32(c["A_log"]),
                                             f32(c["B"]), f32(c["C"]), D=f32(c["D"]),
                                             delta_softplus=False)
            fin = st
        torch.cuda.synchronize()
        np.testing.assert_allclose(to_np(out), c["y"], rtol=2e-6, atol=2e-6)
        np.testing.assert_allclose(to_np(fin), c["final"], rtol=2e-6, atol=2e-6)
