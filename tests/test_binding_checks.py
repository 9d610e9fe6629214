"""The Python binding's own checks: tensors on the host, a caller's workspace
that is not contiguous uint8 on the call's device, and a decode step's output
buffer of the wrong shape are rejected before anything reaches libmss.

On the CPU the library is replaced by a stub that fails the test if any of its
functions is called; on the GPU the same calls are made with device inputs and
one bad buffer each, and must raise before a launch.
"""

import pytest

import mamba_selective_scan_amd as mss
from mamba_selective_scan_amd import _lib


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"libmss.{name} was reached")


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(_lib, "lib", lambda *a, **k: _NoCalls())


def _scan_inputs(device, bsz=1, dim=8, seqlen=16, dstate=4):
    import torch
    g = torch.Generator().manual_seed(0)
    u = torch.randn(bsz, dim, seqlen, generator=g)
    x = dict(u=u, delta_raw=torch.randn(bsz, dim, seqlen, generator=g) * 0.1,
             A_log=torch.zeros(dim, dstate), B=torch.randn(bsz, dstate, seqlen, generator=g),
             C=torch.randn(bsz, dstate, seqlen, generator=g))
    return {k: v.to(device) for k, v in x.items()}


def test_host_tensors_are_rejected(no_library):
    import torch
    x = _scan_inputs("cpu")
    args = (x["u"], x["delta_raw"], x["A_log"], x["B"], x["C"])
    with pytest.raises(ValueError, match="on a GPU"):
        mss.selective_scan_fwd(*args)
    with pytest.raises(ValueError, match="on a GPU"):
        mss.selective_scan_bwd(*args, torch.randn_like(x["u"]))
    with pytest.raises(ValueError, match="on a GPU"):
        mss.selective_scan_fwd_complex(x["u"], x["delta_raw"], x["A_log"], x["A_log"],
                                       x["B"].to(torch.complex64), x["C"].to(torch.complex64))
    state = torch.zeros(1, 8, 4)
    with pytest.raises(ValueError, match="on a GPU"):
        mss.selective_state_update(state, x["u"][:, :, 0], x["delta_raw"][:, :, 0], x["A_log"],
                                   x["B"][:, :, 0], x["C"][:, :, 0])
    w = torch.zeros(8, 4)
    with pytest.raises(ValueError, match="on a GPU"):
        mss.causal_conv1d_fwd(x["u"], w)
    with pytest.raises(ValueError, match="on a GPU"):
        mss.causal_conv1d_update(torch.zeros(1, 8, 3), x["u"][:, :, 0], w)


@pytest.mark.gpu
def test_bad_buffers_are_rejected_before_launch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    dev = torch.device("cuda", 0)
    # 8 channels x 4096 steps is cut into time segments: the call needs a workspace
    x = _scan_inputs(dev, dim=8, seqlen=4096)
    args = (x["u"], x["delta_raw"], x["A_log"], x["B"], x["C"])
    need = mss.scan_workspace_size(x["u"], x["A_log"])
    assert need > 0
    bad = {
        "host": torch.empty(need, dtype=torch.uint8),
        "dtype": torch.empty(need // 4 + 1, dtype=torch.float32, device=dev),
        "strided": torch.empty(2 * need, dtype=torch.uint8, device=dev)[::2],
    }
    for name, ws in bad.items():
        with pytest.raises(ValueError, match="workspace"):
            mss.selective_scan_fwd(*args, workspace=ws)
        with pytest.raises(ValueError, match="workspace"):
            mss.selective_scan_bwd(*args, torch.randn_like(x["u"]), workspace=ws)
    u_t, dr_t = x["u"][:, :, 0], x["delta_raw"][:, :, 0]
    state = torch.zeros(1, 8, 4, device=dev)
    for out in (torch.empty(1, 4, device=dev), torch.empty(1, 8, dtype=torch.bfloat16, device=dev),
                torch.empty(1, 8)):
        with pytest.raises(ValueError, match="out must match"):
            mss.selective_state_update(state, u_t, dr_t, x["A_log"], x["B"][:, :, 0],
                                       x["C"][:, :, 0], out=out)
        with pytest.raises(ValueError, match="out must match"):
            mss.causal_conv1d_update(torch.zeros(1, 8, 3, device=dev), u_t,
                                     torch.zeros(8, 4, device=dev), out=out)
    torch.cuda.synchronize()
