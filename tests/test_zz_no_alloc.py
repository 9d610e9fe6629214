"""The no-allocation forward (mss_selective_scan_fwd_noalloc) against the
forward with a caller's workspace (mss_selective_scan_fwd).

Both run the same kernels on the same inputs, so their outputs, final states
and chunk states must agree bit for bit.  Shapes are chosen so that the
library's scratch array is really used: few channels and a long sequence
(time segments: aggregates and carries in the scratch) and a length that is
not a whole number of 4-step vectors (the ragged-tail state hand-off).  Two
or more calls run back to back, each later one on a smaller problem, so a
call that read anything a previous call left in the scratch would show.
"""

import pytest

from gpu_util import device, note
from mamba_selective_scan_amd.inputs import generate, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _pair(mss, batch, dim, seqlen, layout="bdl", io="f32", seed=0, h0=False):
    """Run both entry points on one problem and require equal results."""
    import torch
    note(f"noalloc vs workspace: B={batch} D={dim} L={seqlen} {layout} {io} h0={h0}")
    x = generate(batch, dim, seqlen, 16, layout, seed=seed)
    dx = to_torch(x, device(), io)
    init = None
    if h0:
        g = torch.Generator().manual_seed(seed + 1)
        init = torch.randn(batch, dim, 16, generator=g).to(device())
    ws_need = mss.scan_workspace_size(dx["u"], dx["A_log"])
    args = (dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"])
    kw = dict(D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], initial_state=init)
    ref_out, ref_fin, ref_cs = mss.selective_scan_fwd(*args, **kw, return_final_state=True,
                                                      return_chunk_states=True)
    out = torch.full_like(dx["u"], float("nan"))
    fin = torch.full((batch, dim, 16), float("nan"), device=device())
    cs = torch.full(mss.chunk_states_shape(dx["u"]), float("nan"), device=device())
    got = mss.selective_scan_fwd_noalloc(*args, **kw, out=out, final_state=fin, chunk_states=cs)
    torch.cuda.synchronize()
    assert got is out
    assert torch.equal(out, ref_out), "out differs"
    assert torch.equal(fin, ref_fin), "final state differs"
    assert torch.equal(cs, ref_cs), "chunk states differ"
    return ws_need


def test_two_calls_second_smaller(mss):
    # segmented with a ragged tail, then a smaller segmented problem with a tail
    assert _pair(mss, 1, 1536, 2051, seed=0) > 0
    assert _pair(mss, 1, 256, 999, seed=1, h0=True) > 0


def test_sequence_of_layouts_and_dtypes(mss):
    # channel-last segmented (cooperative rows), bf16 with a tail, then a shape
    # that needs no scratch at all, then a small segmented one again
    assert _pair(mss, 1, 256, 20003, layout="bld", seed=2) > 0
    assert _pair(mss, 2, 96, 3001, io="bf16", seed=3, h0=True) > 0
    assert _pair(mss, 4, 4096, 64, seed=4) == 0
    assert _pair(mss, 1, 64, 515, seed=5) > 0


def test_aggregate_parts(mss):
    # 1x8192x1117: the aggregate pass in two parts per segment (its part
    # aggregates fill the scratch), both layouts, then a smaller shape
    assert _pair(mss, 1, 8192, 1117, seed=8, h0=True) > 0
    assert _pair(mss, 1, 8192, 1117, layout="bld", seed=9) > 0
    assert _pair(mss, 1, 256, 999, seed=10) > 0


def test_reverse_time(mss):
    import torch
    note("noalloc reverse time")
    x = generate(1, 128, 4097, 16, seed=6)
    dx = to_torch(x, device(), "f32")
    args = (dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"])
    kw = dict(D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], reverse=True)
    ref_out, ref_fin = mss.selective_scan_fwd(*args, **kw, return_final_state=True)
    out = torch.empty_like(dx["u"])
    fin = torch.empty(1, 128, 16, device=device())
    mss.selective_scan_fwd_noalloc(*args, **kw, out=out, final_state=fin)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)


def test_shape_beyond_scratch_is_rejected(mss):
    """A ragged length over more (batch, channel) pairs than the scratch holds
    a tail hand-off for: a typed error before any launch, output untouched."""
    import torch
    from mamba_selective_scan_amd import MssError, _lib
    dim = _lib.MSS_NOALLOC_SCRATCH_BYTES // (16 * 4) + 8
    note(f"noalloc beyond scratch: D={dim} L=3")
    x = generate(1, dim, 3, 16, seed=7)
    dx = to_torch(x, device(), "f32")
    assert mss.scan_workspace_size(dx["u"], dx["A_log"]) > _lib.MSS_NOALLOC_SCRATCH_BYTES
    out = torch.zeros_like(dx["u"])
    with pytest.raises(MssError) as e:
        mss.selective_scan_fwd_noalloc(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                       D=dx["D"], out=out)
    assert e.value.name == "MSS_ERR_SCRATCH_LIMIT"
    torch.cuda.synchronize()
    assert not out.any()


def test_graph_capture_and_replay(mss):
    """The callers this entry point is for record it: captured once in a HIP
    graph (after a first eager call on the device), then replayed with new
    inputs copied into the recorded buffers and unrelated eager work between
    the replays; every replay equals the eager workspace forward bit for bit."""
    import torch
    note("noalloc graph capture")
    shape = (1, 256, 999)  # time segments and a ragged tail: the scratch holds both
    sets = [to_torch(generate(*shape, 16, seed=s), device(), "f32") for s in (11, 12, 13)]
    static = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in sets[0].items()}
    out = torch.empty_like(static["u"])
    fin = torch.empty(shape[0], shape[1], 16, device=device())
    args = lambda d: (d["u"], d["delta_raw"], d["A_log"], d["B"], d["C"])  # noqa: E731
    kw = lambda d: dict(D=d["D"], z=d["z"], dt_bias=d["dt_bias"])  # noqa: E731
    mss.selective_scan_fwd_noalloc(*args(static), **kw(static), out=out, final_state=fin)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mss.selective_scan_fwd_noalloc(*args(static), **kw(static), out=out, final_state=fin)
    torch.cuda.synchronize()
    for rep in range(3):
        src = sets[rep % len(sets)]
        for k in ("u", "delta_raw", "z", "B", "C", "A_log", "D", "dt_bias"):
            static[k].copy_(src[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_fin = mss.selective_scan_fwd(*args(src), **kw(src), return_final_state=True)
        # unrelated eager work on the same GPU between replays
        mss.selective_scan_fwd_noalloc(*args(sets[2]), **kw(sets[2]),
                                       out=torch.empty_like(sets[2]["u"]))
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: out differs"
        assert torch.equal(fin, ref_fin), f"replay {rep}: final state differs"
