"""mamba_selective_scan_amd -- Mamba selective-scan forward and state update, and
the causal depthwise conv1d (+ SiLU) that feeds the scan with its decode step,
on MI355X (gfx950), through the C ABI of libmss (include/mss.h).

This module marshals arguments only: it reads tensor pointers, logical strides
and torch's current HIP stream and calls libmss, whose HIP kernels do every
step of the computation.  PyTorch supplies device memory and streams.  There
is no CPU or PyTorch fallback; without the built library every call raises.

    out = selective_scan_fwd(u, delta_raw, A_log, B, C, D, z, dt_bias)
    out, h = selective_scan_fwd(..., return_final_state=True)
    y = selective_state_update(state, u_t, delta_raw_t, A_log, B_t, C_t, D, z_t, dt_bias)
    u = causal_conv1d_fwd(x, weight, bias)                  # silu(causal conv)
    u, window = causal_conv1d_fwd(x, weight, bias, return_final_state=True)
    u_t = causal_conv1d_update(window, x_t, weight, bias)   # window slides in place
    g = selective_scan_bwd(u, delta_raw, A_log, B, C, dout, D, z, dt_bias)  # dict of grads
    out = selective_scan(u, delta_raw, A_log, B, C, D, z, dt_bias)  # autograd: fwd + bwd

Shapes (logical index order, any strides): u, delta_raw, z, out [B, D, L];
B, C [B, N, L]; A_log [D, N]; D, dt_bias [D]; states [B, D, N] (fp32,
contiguous).  A channel-last [B, L, D] buffer is passed as its transpose(1, 2)
view.  u, delta_raw, z, B, C share one dtype (float32 or bfloat16); A_log, D,
dt_bias and the states are float32.  The conv takes x, out [B, D, L] (any
strides), weight [D, W] fp32 (W <= 4; a [D, 1, W] or [D, W, 1] weight is
viewed as [D, W]), bias [D] fp32, and windows [B, D, W-1] of x's dtype.
"""

from __future__ import annotations

import ctypes

from . import _lib
from ._lib import MSS_MAX_DSTATE, MssError

__all__ = ["selective_scan_fwd", "selective_scan_fwd_noalloc", "selective_state_update", "scan_workspace_size",
           "causal_conv1d_fwd", "causal_conv1d_update", "selective_scan_bwd",
           "scan_bwd_workspace_size", "selective_scan", "selective_scan_fwd_complex",
           "scan_complex_workspace_size", "MssError", "MSS_MAX_DSTATE",
           "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _io_dtype(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return _lib.MSS_F32
    if t.dtype == torch.bfloat16:
        return _lib.MSS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: expected float32 or bfloat16")


def _need(t, name, ndim, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _need_gpu(t, name):
    """The tensor that fixes a call's device must live on a GPU: the kernels
    read and write every pointer from the device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (torch device type 'cuda'), got {t.device}")


def _workspace(t, device):
    """A caller's workspace: contiguous uint8 on the call's device (its byte
    count is passed on; the library checks it against what the call needs)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if t.dtype != torch.uint8 or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return t


def _out_like(out, ref, name):
    """A caller's output buffer for a decode step: the shape, dtype and device
    of ``ref`` (any strides)."""
    if tuple(out.shape) != tuple(ref.shape) or out.dtype != ref.dtype or out.device != ref.device:
        raise ValueError(f"out must match {name} in shape, dtype and device")
    return out


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t, n):
    arr = (ctypes.c_int64 * n)()
    if t is not None:
        for i, s in enumerate(t.stride()):
            arr[i] = s
    return arr


def _contig_f32(t, name, shape, device):
    torch = _torch()
    if t is None:
        return None
    _need(t, name, len(shape), torch.float32, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_handle(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _launch(fn, args, device):
    """Call a library entry point on torch's current stream of ``device``, with
    ``device`` current: torch's default stream is HIP's null stream, which
    stands for the current device's."""
    torch = _torch()
    if device.index is None or device.index == torch.cuda.current_device():
        _lib.check(fn(ctypes.byref(args), _stream_handle(device)))
        return
    with torch.cuda.device(device):
        _lib.check(fn(ctypes.byref(args), _stream_handle(device)))


def _scan_args(u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state, out, final_state,
               delta_softplus, reverse=False):
    torch = _torch()
    _need_gpu(u, "u")
    dev = u.device
    _need(u, "u", 3)
    bsz, dim, seqlen = u.shape
    dt = u.dtype
    _need(delta_raw, "delta_raw", 3, dt, dev)
    _need(B, "B", 3, dt, dev)
    _need(C, "C", 3, dt, dev)
    _need(A_log, "A_log", 2, torch.float32, dev)
    dstate = A_log.shape[1]
    if tuple(delta_raw.shape) != (bsz, dim, seqlen):
        raise ValueError("delta_raw must have the shape of u")
    if tuple(B.shape) != (bsz, dstate, seqlen) or tuple(C.shape) != (bsz, dstate, seqlen):
        raise ValueError(f"B and C must have shape {(bsz, dstate, seqlen)}")
    if tuple(A_log.shape) != (dim, dstate):
        raise ValueError(f"A_log must have shape {(dim, dstate)}")
    if z is not None:
        _need(z, "z", 3, dt, dev)
        if tuple(z.shape) != (bsz, dim, seqlen):
            raise ValueError("z must have the shape of u")
    _contig_f32(D, "D", (dim,), dev)
    _contig_f32(dt_bias, "dt_bias", (dim,), dev)
    _contig_f32(initial_state, "initial_state", (bsz, dim, dstate), dev)
    a = _lib.new_scan_args()
    a.io_dtype = _io_dtype(u)
    a.batch, a.dim, a.seqlen, a.dstate = bsz, dim, seqlen, dstate
    a.u, a.u_stride = _ptr(u), _strides(u, 3)
    a.delta_raw, a.delta_stride = _ptr(delta_raw), _strides(delta_raw, 3)
    a.A_log, a.A_log_stride = _ptr(A_log), _strides(A_log, 2)
    a.B, a.B_stride = _ptr(B), _strides(B, 3)
    a.C, a.C_stride = _ptr(C), _strides(C, 3)
    a.D = _ptr(D)
    a.z, a.z_stride = _ptr(z), _strides(z, 3)
    a.dt_bias = _ptr(dt_bias)
    a.initial_state = _ptr(initial_state)
    a.out, a.out_stride = _ptr(out), _strides(out, 3)
    a.final_state = _ptr(final_state)
    a.delta_softplus = 1 if delta_softplus else 0
    a.reverse = 1 if reverse else 0
    return a


def scan_workspace_size(u, A_log) -> int:
    """Workspace bytes selective_scan_fwd needs for u [B, D, L] and A_log [D, N]."""
    a = _lib.new_scan_args()
    a.io_dtype = _io_dtype(u)
    a.batch, a.dim, a.seqlen = u.shape
    a.dstate = A_log.shape[1]
    st = ctypes.c_int(0)
    n = _lib.lib().mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
    _lib.check(st.value)
    return int(n)


def chunk_states_shape(u):
    """Shape of the chunk-state array for u [B, D, L]: (ceil(L / 16), B, D, 16),
    fp32 -- the state entering every 16-step chunk of logical time, 16 slots
    per channel (slots n >= dstate hold 0)."""
    bsz, dim, seqlen = u.shape
    q = (seqlen + _lib.MSS_STATE_CHUNK - 1) // _lib.MSS_STATE_CHUNK
    return (q, bsz, dim, _lib.MSS_MAX_DSTATE)


def selective_scan_fwd(u, delta_raw, A_log, B, C, D=None, z=None, dt_bias=None, *,
                       delta_softplus=True, initial_state=None, return_final_state=False,
                       out=None, final_state=None, workspace=None, reverse=False,
                       return_chunk_states=False, chunk_states=None, _noalloc=False):
    """Selective-scan forward on u's device, ordered on torch's current stream.

    ``reverse=True`` runs the recurrence from the last step to the first (the
    second direction of a bidirectional layer) on the same buffers.

    Returns ``out`` (shape and layout of u), followed by the fp32 state
    [B, D, N] after the last step when ``return_final_state`` and by the chunk
    states (chunk_states_shape(u), for selective_scan_bwd) when
    ``return_chunk_states``.  ``out``, ``final_state``, ``chunk_states`` and
    ``workspace`` (uint8, at least scan_workspace_size bytes) may be supplied
    to avoid allocation.
    """
    torch = _torch()
    lib = _lib.lib()
    if out is None:
        out = torch.empty_like(u)
    if return_final_state and final_state is None:
        final_state = torch.empty((u.shape[0], u.shape[1], A_log.shape[1]), dtype=torch.float32,
                                  device=u.device)
    if final_state is not None:
        _contig_f32(final_state, "final_state", (u.shape[0], u.shape[1], A_log.shape[1]), u.device)
    if return_chunk_states and chunk_states is None:
        chunk_states = torch.empty(chunk_states_shape(u), dtype=torch.float32, device=u.device)
    if chunk_states is not None:
        _contig_f32(chunk_states, "chunk_states", chunk_states_shape(u), u.device)
    a = _scan_args(u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state, out, final_state,
                   delta_softplus, reverse)
    a.chunk_states = _ptr(chunk_states)
    if tuple(out.shape) != tuple(u.shape) or out.dtype != u.dtype or out.device != u.device:
        raise ValueError("out must match u in shape, dtype and device")
    if _noalloc:
        if workspace is not None:
            raise ValueError("the no-allocation forward takes no workspace")
        _launch(lib.mss_selective_scan_fwd_noalloc, a, u.device)
    else:
        st = ctypes.c_int(0)
        need = lib.mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
        _lib.check(st.value)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
        a.workspace = _ptr(_workspace(workspace, u.device))
        a.workspace_bytes = workspace.numel() * workspace.element_size()
        _launch(lib.mss_selective_scan_fwd, a, u.device)
    res = (out,) + ((final_state,) if return_final_state else ()) + \
        ((chunk_states,) if return_chunk_states else ())
    return res if len(res) > 1 else out


def selective_scan_fwd_noalloc(u, delta_raw, A_log, B, C, D=None, z=None, dt_bias=None, *,
                               delta_softplus=True, initial_state=None, out=None,
                               final_state=None, reverse=False, chunk_states=None):
    """selective_scan_fwd through mss_selective_scan_fwd_noalloc: the library
    allocates nothing and takes no workspace (its scratch is a per-GPU device
    array of MSS_NOALLOC_SCRATCH_BYTES that all such calls on a GPU share, so
    calls on one GPU must not overlap in time).  Without ``out`` this binding
    allocates it from torch; pass ``out`` (and ``final_state`` /
    ``chunk_states`` when wanted) for a call that allocates nothing at all.
    Returns ``out``."""
    return selective_scan_fwd(u, delta_raw, A_log, B, C, D, z, dt_bias,
                              delta_softplus=delta_softplus, initial_state=initial_state,
                              out=out, final_state=final_state, reverse=reverse,
                              chunk_states=chunk_states, _noalloc=True)


def scan_complex_workspace_size(u, A_log) -> int:
    """Workspace bytes selective_scan_fwd_complex needs for u [B, D, L] and
    A_log [D, N] (0 unless the shape is cut into time segments)."""
    a = _lib.new_scan_complex_args()
    a.batch, a.dim, a.seqlen = u.shape
    a.dstate = A_log.shape[1]
    st = ctypes.c_int(0)
    n = _lib.lib().mss_selective_scan_fwd_complex_workspace_size(ctypes.byref(a), ctypes.byref(st))
    _lib.check(st.value)
    return int(n)


def selective_scan_fwd_complex(u, delta_raw, A_log, A_imag, B, C, D=None, z=None, dt_bias=None, *,
                               delta_softplus=True, initial_state=None,
                               return_final_state=False, out=None, final_state=None,
                               workspace=None):
    """Selective-scan forward with complex A = -exp(A_log) + i A_imag, ordered on
    torch's current stream.

    u, delta_raw, z: fp32 [B, D, L]; A_log, A_imag: fp32 [D, N]; B, C:
    complex64 [B, N, L] (any strides); initial_state, final_state: complex64
    [B, D, N] contiguous.  Returns ``out`` (fp32, the real part of C . h plus
    D u, gated), or ``(out, final_state)`` when ``return_final_state``.
    ``workspace`` (uint8, at least scan_complex_workspace_size bytes) may be
    supplied to avoid its allocation.
    """
    torch = _torch()
    lib = _lib.lib()
    _need_gpu(u, "u")
    dev = u.device
    _need(u, "u", 3, torch.float32, dev)
    bsz, dim, seqlen = u.shape
    _need(delta_raw, "delta_raw", 3, torch.float32, dev)
    _need(A_log, "A_log", 2, torch.float32, dev)
    _need(A_imag, "A_imag", 2, torch.float32, dev)
    dstate = A_log.shape[1]
    _need(B, "B", 3, torch.complex64, dev)
    _need(C, "C", 3, torch.complex64, dev)
    if tuple(delta_raw.shape) != (bsz, dim, seqlen):
        raise ValueError("delta_raw must have the shape of u")
    if tuple(A_log.shape) != (dim, dstate) or tuple(A_imag.shape) != (dim, dstate):
        raise ValueError(f"A_log and A_imag must have shape {(dim, dstate)}")
    if tuple(B.shape) != (bsz, dstate, seqlen) or tuple(C.shape) != (bsz, dstate, seqlen):
        raise ValueError(f"B and C must have shape {(bsz, dstate, seqlen)}")
    if z is not None:
        _need(z, "z", 3, torch.float32, dev)
        if tuple(z.shape) != (bsz, dim, seqlen):
            raise ValueError("z must have the shape of u")
    _contig_f32(D, "D", (dim,), dev)
    _contig_f32(dt_bias, "dt_bias", (dim,), dev)
    for t, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _need(t, name, 3, torch.complex64, dev)
            if tuple(t.shape) != (bsz, dim, dstate) or not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous with shape {(bsz, dim, dstate)}")
    if out is None:
        out = torch.empty_like(u)
    if return_final_state and final_state is None:
        final_state = torch.empty((bsz, dim, dstate), dtype=torch.complex64, device=dev)
    if tuple(out.shape) != tuple(u.shape) or out.dtype != torch.float32 or out.device != dev:
        raise ValueError("out must be fp32 with the shape of u on its device")
    a = _lib.new_scan_complex_args()
    a.batch, a.dim, a.seqlen, a.dstate = bsz, dim, seqlen, dstate
    a.u, a.u_stride = _ptr(u), _strides(u, 3)
    a.delta_raw, a.delta_stride = _ptr(delta_raw), _strides(delta_raw, 3)
    a.A_log, a.A_log_stride = _ptr(A_log), _strides(A_log, 2)
    a.A_imag, a.A_imag_stride = _ptr(A_imag), _strides(A_imag, 2)
    a.B, a.B_stride = _ptr(B), _strides(B, 3)
    a.C, a.C_stride = _ptr(C), _strides(C, 3)
    a.D = _ptr(D)
    a.z, a.z_stride = _ptr(z), _strides(z, 3)
    a.dt_bias = _ptr(dt_bias)
    a.initial_state = _ptr(initial_state)
    a.out, a.out_stride = _ptr(out), _strides(out, 3)
    a.final_state = _ptr(final_state)
    a.delta_softplus = 1 if delta_softplus else 0
    st = ctypes.c_int(0)
    need = lib.mss_selective_scan_fwd_complex_workspace_size(ctypes.byref(a), ctypes.byref(st))
    _lib.check(st.value)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        a.workspace = _ptr(_workspace(workspace, dev))
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _launch(lib.mss_selective_scan_fwd_complex, a, dev)
    return (out, final_state) if return_final_state else out


def selective_state_update(state, u, delta_raw, A_log, B, C, D=None, z=None, dt_bias=None, *,
                           delta_softplus=True, out=None):
    """One decode step: updates ``state`` [B, D, N] (fp32, contiguous) in place and
    returns out [B, D].  u, delta_raw, z are [B, D]; B, C are [B, N]."""
    torch = _torch()
    lib = _lib.lib()
    _need_gpu(state, "state")
    dev = state.device
    _need(state, "state", 3, torch.float32, dev)
    if not state.is_contiguous():
        raise ValueError("state must be contiguous")
    bsz, dim, dstate = state.shape
    _need(u, "u", 2, None, dev)
    dt = u.dtype
    _need(delta_raw, "delta_raw", 2, dt, dev)
    _need(B, "B", 2, dt, dev)
    _need(C, "C", 2, dt, dev)
    _need(A_log, "A_log", 2, torch.float32, dev)
    if tuple(u.shape) != (bsz, dim) or tuple(delta_raw.shape) != (bsz, dim):
        raise ValueError(f"u and delta_raw must have shape {(bsz, dim)}")
    if tuple(B.shape) != (bsz, dstate) or tuple(C.shape) != (bsz, dstate):
        raise ValueError(f"B and C must have shape {(bsz, dstate)}")
    if tuple(A_log.shape) != (dim, dstate):
        raise ValueError(f"A_log must have shape {(dim, dstate)}")
    if z is not None:
        _need(z, "z", 2, dt, dev)
    _contig_f32(D, "D", (dim,), dev)
    _contig_f32(dt_bias, "dt_bias", (dim,), dev)
    out = torch.empty_like(u) if out is None else _out_like(out, u, "u")
    a = _lib.new_step_args()
    a.io_dtype = _io_dtype(u)
    a.batch, a.dim, a.dstate = bsz, dim, dstate
    a.state = _ptr(state)
    a.u, a.u_stride = _ptr(u), _strides(u, 2)
    a.delta_raw, a.delta_stride = _ptr(delta_raw), _strides(delta_raw, 2)
    a.A_log, a.A_log_stride = _ptr(A_log), _strides(A_log, 2)
    a.B, a.B_stride = _ptr(B), _strides(B, 2)
    a.C, a.C_stride = _ptr(C), _strides(C, 2)
    a.D = _ptr(D)
    a.z, a.z_stride = _ptr(z), _strides(z, 2)
    a.dt_bias = _ptr(dt_bias)
    a.out, a.out_stride = _ptr(out), _strides(out, 2)
    a.delta_softplus = 1 if delta_softplus else 0
    _launch(lib.mss_selective_state_update, a, dev)
    return out


_ACTIVATIONS = {None: _lib.MSS_ACT_NONE, "none": _lib.MSS_ACT_NONE, "silu": _lib.MSS_ACT_SILU}


def _conv_weight(weight, dim, device):
    torch = _torch()
    _need(weight, "weight", weight.dim(), torch.float32, device)
    if weight.dim() == 3:
        if weight.shape[1] == 1:
            weight = weight[:, 0, :]
        elif weight.shape[2] == 1:
            weight = weight[:, :, 0]
        else:
            raise ValueError(f"a 3-d conv weight must be [D, 1, W] or [D, W, 1], got "
                             f"{tuple(weight.shape)}")
    if weight.dim() != 2 or weight.shape[0] != dim:
        raise ValueError(f"weight must be [{dim}, W], got {tuple(weight.shape)}")
    return weight


def _window(t, name, shape, dtype, device):
    if t is None:
        return None
    _need(t, name, 3, dtype, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def causal_conv1d_fwd(x, weight, bias=None, *, activation="silu", initial_state=None,
                      return_final_state=False, out=None, final_state=None):
    """Causal depthwise conv1d with optional SiLU, ordered on torch's current stream.

    x [B, D, L] (float32 or bfloat16, any strides); weight [D, W] fp32;
    bias [D] fp32 or None; activation "silu" or None; initial_state
    [B, D, W-1] (x's dtype, contiguous) is the window before the first step
    (None means zeros).  Returns out (x's shape and dtype), or
    (out, final_state) with the window after the last step when
    ``return_final_state``.
    """
    torch = _torch()
    lib = _lib.lib()
    _need_gpu(x, "x")
    dev = x.device
    _need(x, "x", 3)
    bsz, dim, seqlen = x.shape
    weight = _conv_weight(weight, dim, dev)
    width = weight.shape[1]
    _contig_f32(bias, "bias", (dim,), dev)
    if activation not in _ACTIVATIONS:
        raise ValueError(f"activation must be 'silu' or None, got {activation!r}")
    win_shape = (bsz, dim, width - 1)
    _window(initial_state, "initial_state", win_shape, x.dtype, dev)
    if out is None:
        out = torch.empty_like(x)
    if tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype or out.device != dev:
        raise ValueError("out must match x in shape, dtype and device")
    if return_final_state and final_state is None:
        final_state = torch.empty(win_shape, dtype=x.dtype, device=dev)
    _window(final_state, "final_state", win_shape, x.dtype, dev)
    a = _lib.new_conv_args()
    a.io_dtype = _io_dtype(x)
    a.batch, a.dim, a.seqlen, a.width = bsz, dim, seqlen, width
    a.x, a.x_stride = _ptr(x), _strides(x, 3)
    a.weight, a.weight_stride = _ptr(weight), _strides(weight, 2)
    a.bias = _ptr(bias)
    a.initial_state = _ptr(initial_state)
    a.out, a.out_stride = _ptr(out), _strides(out, 3)
    a.final_state = _ptr(final_state)
    a.activation = _ACTIVATIONS[activation]
    _launch(lib.mss_causal_conv1d_fwd, a, dev)
    if return_final_state:
        return out, final_state
    return out


def causal_conv1d_update(state, x, weight, bias=None, *, activation="silu", out=None):
    """One conv1d decode step: returns out [B, D] for the new sample x [B, D] and
    slides ``state`` [B, D, W-1] (x's dtype, contiguous) in place."""
    torch = _torch()
    lib = _lib.lib()
    _need_gpu(x, "x")
    dev = x.device
    _need(x, "x", 2)
    bsz, dim = x.shape
    weight = _conv_weight(weight, dim, dev)
    width = weight.shape[1]
    _contig_f32(bias, "bias", (dim,), dev)
    if activation not in _ACTIVATIONS:
        raise ValueError(f"activation must be 'silu' or None, got {activation!r}")
    _window(state, "state", (bsz, dim, width - 1), x.dtype, dev)
    out = torch.empty_like(x) if out is None else _out_like(out, x, "x")
    a = _lib.new_conv_step_args()
    a.io_dtype = _io_dtype(x)
    a.batch, a.dim, a.width = bsz, dim, width
    a.state = _ptr(state) if width > 1 else None
    a.x, a.x_stride = _ptr(x), _strides(x, 2)
    a.weight, a.weight_stride = _ptr(weight), _strides(weight, 2)
    a.bias = _ptr(bias)
    a.out, a.out_stride = _ptr(out), _strides(out, 2)
    a.activation = _ACTIVATIONS[activation]
    _launch(lib.mss_causal_conv1d_update, a, dev)
    return out


def _bwd_shape_args(u, A_log):
    a = _lib.new_scan_bwd_args()
    a.io_dtype = _io_dtype(u)
    a.batch, a.dim, a.seqlen = u.shape
    a.dstate = A_log.shape[1]
    return a


def scan_bwd_workspace_size(u, A_log) -> int:
    """Workspace bytes selective_scan_bwd needs for u [B, D, L] and A_log [D, N]."""
    a = _bwd_shape_args(u, A_log)
    st = ctypes.c_int(0)
    n = _lib.lib().mss_selective_scan_bwd_workspace_size(ctypes.byref(a), ctypes.byref(st))
    _lib.check(st.value)
    return int(n)


def selective_scan_bwd(u, delta_raw, A_log, B, C, dout, D=None, z=None, dt_bias=None, *,
                       delta_softplus=True, initial_state=None, dfinal_state=None,
                       workspace=None, reverse=False, chunk_states=None):
    """Backward of selective_scan_fwd, ordered on torch's current stream.

    dout has u's shape and dtype; dfinal_state [B, D, N] fp32 (optional) is the
    gradient reaching the exported final state.  Returns a dict with du,
    ddelta_raw, dB, dC (dtype of u, shapes of the inputs), dA_log [D, N] fp32,
    and dD, dz, ddt_bias, dinitial_state for the optional inputs that are given.
    ``reverse`` must match the forward's.  ``chunk_states``, recorded by
    selective_scan_fwd on the same inputs and flags, saves the backward its own
    forward pass over the sequence.
    """
    torch = _torch()
    lib = _lib.lib()
    a = _scan_args(u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state, None, None,
                   delta_softplus, reverse)
    dev = u.device
    _need(dout, "dout", 3, u.dtype, dev)
    if tuple(dout.shape) != tuple(u.shape):
        raise ValueError("dout must have the shape of u")
    bsz, dim, _ = u.shape
    dstate = A_log.shape[1]
    _contig_f32(dfinal_state, "dfinal_state", (bsz, dim, dstate), dev)
    if chunk_states is not None:
        _contig_f32(chunk_states, "chunk_states", chunk_states_shape(u), dev)
    g = {
        "du": torch.empty_like(u), "ddelta_raw": torch.empty_like(delta_raw),
        "dA_log": torch.empty((dim, dstate), dtype=torch.float32, device=dev),
        "dB": torch.empty_like(B), "dC": torch.empty_like(C),
        "dD": torch.empty_like(D) if D is not None else None,
        "dz": torch.empty_like(z) if z is not None else None,
        "ddt_bias": torch.empty_like(dt_bias) if dt_bias is not None else None,
        "dinitial_state": (torch.empty_like(initial_state) if initial_state is not None
                           else None),
    }
    b = _lib.new_scan_bwd_args()
    for name, *_ in _lib.ScanArgs._fields_:
        if hasattr(b, name) and name not in ("struct_size", "out", "out_stride", "final_state",
                                            "chunk_states", "workspace", "workspace_bytes"):
            setattr(b, name, getattr(a, name))
    b.struct_size = ctypes.sizeof(_lib.ScanBwdArgs)
    b.dout, b.dout_stride = _ptr(dout), _strides(dout, 3)
    b.dfinal_state = _ptr(dfinal_state)
    b.chunk_states = _ptr(chunk_states)
    b.du, b.du_stride = _ptr(g["du"]), _strides(g["du"], 3)
    b.ddelta_raw, b.ddelta_stride = _ptr(g["ddelta_raw"]), _strides(g["ddelta_raw"], 3)
    b.dA_log = _ptr(g["dA_log"])
    b.dB, b.dB_stride = _ptr(g["dB"]), _strides(g["dB"], 3)
    b.dC, b.dC_stride = _ptr(g["dC"]), _strides(g["dC"], 3)
    b.dD = _ptr(g["dD"])
    b.dz, b.dz_stride = _ptr(g["dz"]), _strides(g["dz"], 3)
    b.ddt_bias = _ptr(g["ddt_bias"])
    b.dinitial_state = _ptr(g["dinitial_state"])
    st = ctypes.c_int(0)
    need = lib.mss_selective_scan_bwd_workspace_size(ctypes.byref(b), ctypes.byref(st))
    _lib.check(st.value)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    b.workspace = _ptr(_workspace(workspace, dev))
    b.workspace_bytes = workspace.numel() * workspace.element_size()
    _launch(lib.mss_selective_scan_bwd, b, dev)
    return {k: v for k, v in g.items() if v is not None}


_SCAN_FN = None


def _scan_fn():
    """torch.autograd.Function over selective_scan_fwd / selective_scan_bwd
    (built on first use so that importing this module does not import torch)."""
    global _SCAN_FN
    if _SCAN_FN is not None:
        return _SCAN_FN
    torch = _torch()

    class SelectiveScanFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state,
                    delta_softplus, reverse):
            # the forward records its chunk states, which the backward reads
            # instead of recomputing them
            out, final, states = selective_scan_fwd(u, delta_raw, A_log, B, C, D, z, dt_bias,
                                                    delta_softplus=delta_softplus,
                                                    initial_state=initial_state,
                                                    return_final_state=True,
                                                    return_chunk_states=True, reverse=reverse)
            ctx.save_for_backward(u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state, states)
            ctx.flags = (delta_softplus, reverse)
            return out, final

        @staticmethod
        def backward(ctx, dout, dfinal):
            u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state, states = ctx.saved_tensors
            delta_softplus, reverse = ctx.flags
            if dout is None:
                dout = torch.zeros_like(u)
            # The backward reads dout through its strides (a stride-0 gradient
            # from out.sum() is read as is); the final-state gradient is a
            # contiguous [B, D, N] array in the ABI, and sum() or mean() of the
            # final state hands over an expanded stride-0 view.
            if dfinal is not None:
                dfinal = dfinal.contiguous()
            g = selective_scan_bwd(u, delta_raw, A_log, B, C, dout, D, z, dt_bias,
                                   delta_softplus=delta_softplus, initial_state=initial_state,
                                   dfinal_state=dfinal, reverse=reverse, chunk_states=states)
            return (g["du"], g["ddelta_raw"], g["dA_log"], g["dB"], g["dC"], g.get("dD"),
                    g.get("dz"), g.get("ddt_bias"), g.get("dinitial_state"), None, None)

    _SCAN_FN = SelectiveScanFn
    return _SCAN_FN


def selective_scan(u, delta_raw, A_log, B, C, D=None, z=None, dt_bias=None, *,
                   delta_softplus=True, initial_state=None, reverse=False,
                   return_final_state=False):
    """Selective scan with autograd: the forward of selective_scan_fwd, and on
    ``backward()`` the gradients of every tensor input from selective_scan_bwd
    (including through the final state when it is returned and used)."""
    out, final = _scan_fn().apply(u, delta_raw, A_log, B, C, D, z, dt_bias, initial_state,
                                  delta_softplus, reverse)
    return (out, final) if return_final_state else out
