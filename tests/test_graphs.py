"""Graph capture: every entry point enqueues only kernel launches on the
caller's stream (no allocation, memset, copy or synchronisation inside the
library), so a torch CUDA graph can record it and replay it.  Each test
records a call, replays the graph several times with new inputs copied into
the recorded buffers and with unrelated eager work and synchronisations
between the replays, and requires every replay to equal the eager call on the
same inputs bit for bit (the kernels are deterministic).
"""

import pytest

from gpu_util import device, note
from mamba_selective_scan_amd.inputs import generate, to_torch

pytestmark = pytest.mark.gpu

ACT = ("u", "delta_raw", "z", "B", "C")


@pytest.fixture(scope="module")
def mss():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mamba_selective_scan_amd as m
    return m


def _inputs(batch, dim, seqlen, seed, io="f32", layout="bdl"):
    return to_torch(generate(batch, dim, seqlen, 16, layout, seed=seed), device(), io)


def _clone(dx):
    import torch
    return {k: v.clone() if isinstance(v, torch.Tensor) else v for k, v in dx.items()}


def _load(static, src):
    """Copy the inputs of src (activations and parameters) into the recorded
    input buffers."""
    for k in ACT + ("A_log", "D", "dt_bias"):
        static[k].copy_(src[k])


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


def _noise(mss, dx):
    """Unrelated eager work between replays."""
    import torch
    mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"], D=dx["D"],
                           z=dx["z"], dt_bias=dx["dt_bias"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape,layout", [((1, 1536, 2048), "bdl"), ((2, 200, 1001), "bdl"),
                                          ((1, 256, 3000), "bld")])
def test_forward_replays(mss, shape, layout):
    """Time segments (aggregate, carry and main passes), a ragged tail pass and
    the channel-last layout, each with final state and chunk states."""
    import torch
    batch, dim, seqlen = shape
    note(f"graph forward {shape} {layout}")
    sets = [_inputs(batch, dim, seqlen, s, layout=layout) for s in (1, 2)]
    static = _clone(sets[0])
    out = torch.empty_like(static["u"])
    fin = torch.empty(batch, dim, 16, dtype=torch.float32, device=device())
    cs = torch.empty(mss.chunk_states_shape(static["u"]), dtype=torch.float32, device=device())
    ws = torch.empty(max(mss.scan_workspace_size(static["u"], static["A_log"]), 1),
                     dtype=torch.uint8, device=device())

    def call(dx, o, f, c):
        return mss.selective_scan_fwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                      D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"], out=o,
                                      final_state=f, chunk_states=c, workspace=ws)

    g, _ = _capture(lambda: call(static, out, fin, cs))
    ref = []
    for dx in sets:
        o, f, c = torch.empty_like(out), torch.empty_like(fin), torch.empty_like(cs)
        call(dx, o, f, c)
        ref.append((o, f, c))
    torch.cuda.synchronize()
    for rep, which in enumerate((1, 0, 1)):
        _load(static, sets[which])
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        cs.fill_(float("nan"))
        _noise(mss, sets[1 - which])
        g.replay()
        torch.cuda.synchronize()
        o, f, c = ref[which]
        assert torch.equal(out, o), f"replay {rep}: out differs"
        assert torch.equal(fin, f), f"replay {rep}: final state differs"
        assert torch.equal(cs, c), f"replay {rep}: chunk states differ"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_loop_replays(mss, io):
    """Eight state-update steps recorded as one graph: a decode loop with one
    launch per replay of the whole loop."""
    import torch
    batch, dim, steps = 2, 1536, 8
    note(f"graph decode loop {io}")
    sets = [_inputs(batch, dim, steps, s, io) for s in (3, 4)]
    static = _clone(sets[0])
    g0 = torch.Generator().manual_seed(5)
    s0 = torch.randn(batch, dim, 16, generator=g0).to(device())
    state = s0.clone()
    outs = [torch.empty(batch, dim, dtype=static["u"].dtype, device=device()) for _ in range(steps)]

    def loop(dx, st, os_):
        for t in range(steps):
            mss.selective_state_update(st, dx["u"][:, :, t], dx["delta_raw"][:, :, t], dx["A_log"],
                                       dx["B"][:, :, t], dx["C"][:, :, t], D=dx["D"],
                                       z=dx["z"][:, :, t], dt_bias=dx["dt_bias"], out=os_[t])

    g, _ = _capture(lambda: loop(static, state, outs))
    ref = []
    for dx in sets:
        st = s0.clone()
        os_ = [torch.empty_like(o) for o in outs]
        loop(dx, st, os_)
        ref.append((st, os_))
    torch.cuda.synchronize()
    for rep, which in enumerate((0, 1, 0)):
        _load(static, sets[which])
        state.copy_(s0)
        _noise(mss, sets[1 - which])
        g.replay()
        torch.cuda.synchronize()
        st, os_ = ref[which]
        assert torch.equal(state, st), f"replay {rep}: state differs"
        for t in range(steps):
            assert torch.equal(outs[t], os_[t]), f"replay {rep}: step {t} out differs"


def test_backward_replays(mss):
    """The backward at a time-split shape (segment aggregates and carries), its
    gradients allocated once inside the recorded call."""
    import torch
    batch, dim, seqlen = 1, 1536, 2048
    note("graph backward")
    sets = [_inputs(batch, dim, seqlen, s) for s in (6, 7)]
    for dx in sets:
        dx["dout"] = torch.randn_like(dx["u"])
    static = _clone(sets[0])

    def call(dx):
        return mss.selective_scan_bwd(dx["u"], dx["delta_raw"], dx["A_log"], dx["B"], dx["C"],
                                      dx["dout"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"])

    g, grads = _capture(lambda: call(static))
    ref = [call(dx) for dx in sets]
    torch.cuda.synchronize()
    for rep, which in enumerate((1, 0)):
        _load(static, sets[which])
        static["dout"].copy_(sets[which]["dout"])
        for v in grads.values():
            if v is not None:
                v.fill_(float("nan"))
        _noise(mss, sets[1 - which])
        g.replay()
        torch.cuda.synchronize()
        for k, v in grads.items():
            if v is not None:
                assert torch.equal(v, ref[which][k]), f"replay {rep}: {k} differs"


def test_conv_prefill_and_step_replays(mss):
    """conv1d + SiLU over a sequence with its final window, then one conv
    decode step on that window, recorded as one graph."""
    import torch
    batch, dim, seqlen, width = 2, 512, 777, 4
    note("graph conv")
    g0 = torch.Generator().manual_seed(8)
    sets = [{"x": torch.randn(batch, dim, seqlen, generator=g0).to(device()),
             "x1": torch.randn(batch, dim, generator=g0).to(device())} for _ in range(2)]
    weight = torch.randn(dim, width, generator=g0).to(device())
    bias = torch.randn(dim, generator=g0).to(device())
    static = _clone(sets[0])
    out = torch.empty_like(static["x"])
    win = torch.empty(batch, dim, width - 1, device=device())
    y1 = torch.empty(batch, dim, device=device())

    def call(dx, o, w, y):
        mss.causal_conv1d_fwd(dx["x"], weight, bias, out=o, final_state=w)
        mss.causal_conv1d_update(w, dx["x1"], weight, bias, out=y)

    g, _ = _capture(lambda: call(static, out, win, y1))
    ref = []
    for dx in sets:
        r = (torch.empty_like(out), torch.empty_like(win), torch.empty_like(y1))
        call(dx, *r)
        ref.append(r)
    torch.cuda.synchronize()
    for rep, which in enumerate((1, 0)):
        for k in static:
            static[k].copy_(sets[which][k])
        out.fill_(float("nan"))
        y1.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o, w, y = ref[which]
        assert torch.equal(out, o) and torch.equal(win, w) and torch.equal(y1, y), f"replay {rep}"


def test_complex_forward_replays(mss):
    """The complex-A forward recorded once and replayed with new inputs."""
    import torch
    from mamba_selective_scan_amd.inputs import complex_to_torch, generate_complex
    note("graph complex forward")
    sets = [complex_to_torch(generate_complex(2, 48, 300, 16, seed=s), device()) for s in (9, 10)]
    static = _clone(sets[0])
    out = torch.empty_like(static["u"])
    fin = torch.empty(2, 48, 16, dtype=torch.complex64, device=device())
    keys = ("u", "delta_raw", "z", "B", "C", "A_log", "A_imag", "D", "dt_bias")

    def call(dx, o, f):
        mss.selective_scan_fwd_complex(dx["u"], dx["delta_raw"], dx["A_log"], dx["A_imag"], dx["B"],
                                       dx["C"], D=dx["D"], z=dx["z"], dt_bias=dx["dt_bias"],
                                       out=o, final_state=f, return_final_state=True)

    g, _ = _capture(lambda: call(static, out, fin))
    ref = []
    for dx in sets:
        o, f = torch.empty_like(out), torch.empty_like(fin)
        call(dx, o, f)
        ref.append((o, f))
    torch.cuda.synchronize()
    for rep, which in enumerate((1, 0)):
        for k in keys:
            static[k].copy_(sets[which][k])
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[which][0]) and torch.equal(fin, ref[which][1]), f"replay {rep}"
