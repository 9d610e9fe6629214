"""fp64 CPU oracle for the Mamba selective-scan forward and state update, and
for the causal depthwise conv1d (+ SiLU) that feeds the scan, with its
sliding-window decode step.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product package
(``mamba_selective_scan_amd``) never imports this module, and this module
imports nothing from the product package.

The arithmetic lives in ``mss_oracle.c`` (scan forward and state update),
``mss_oracle_bwd.c`` (the scan's backward), ``mss_oracle_conv.c`` and
``mss_oracle_cplx.c`` (the forward with complex A; B, C and the states are
complex128 there) -- plain C, fp64, sequential in time, OpenMP across
independent channels in the forward.  This wrapper only marshals numpy arrays:
every input is converted exactly to float64 and laid out contiguously as

    u, delta_raw, z, out : [batch, dim, seqlen]
    B, C                 : [batch, dstate, seqlen]
    A_log                : [dim, dstate]
    D, dt_bias           : [dim]
    h0, final_state      : [batch, dim, dstate]
    conv: x, out [batch, dim, seqlen]; w [dim, width]; bias [dim];
          windows (init, final, state) [batch, dim, width - 1]

Values stored in float32 or bfloat16 upcast to float64 without rounding, so the
oracle consumes exactly the bytes the GPU consumes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mss_oracle.c")
SOURCES = {"scan": _SRC, "conv": os.path.join(_HERE, "mss_oracle_conv.c"),
           "bwd": os.path.join(_HERE, "mss_oracle_bwd.c"),
           "cplx": os.path.join(_HERE, "mss_oracle_cplx.c")}
LIB_PATH = os.path.join(_HERE, "libmss_oracle.so")

_lib = None


def build(src: str | None = None, out: str = LIB_PATH, replace: dict | None = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math).

    ``replace`` maps a key of SOURCES to another file to compile in its place
    (the mutation tests build a library with one source file altered);
    ``src`` is shorthand for replacing the scan source.
    """
    srcs = dict(SOURCES)
    if src is not None:
        srcs["scan"] = src
    srcs.update(replace or {})
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", *srcs.values(), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.mss_oracle_softplus.argtypes = [ctypes.c_double]
    lib.mss_oracle_softplus.restype = ctypes.c_double
    lib.mss_oracle_silu.argtypes = [ctypes.c_double]
    lib.mss_oracle_silu.restype = ctypes.c_double
    lib.mss_oracle_max_threads.argtypes = []
    lib.mss_oracle_max_threads.restype = ctypes.c_int
    lib.mss_oracle_scan_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 9 + [
        ctypes.c_int, dp, dp, ctypes.c_int]
    lib.mss_oracle_scan_fwd.restype = ctypes.c_int
    lib.mss_oracle_state_update.argtypes = [i64, i64, i64, dp] + [dp] * 8 + [
        ctypes.c_int, dp]
    lib.mss_oracle_state_update.restype = ctypes.c_int
    lib.mss_oracle_scan_bwd.argtypes = [i64, i64, i64, i64] + [dp] * 9 + [ctypes.c_int] + \
        [dp] * 2 + [dp] * 9
    lib.mss_oracle_scan_bwd.restype = ctypes.c_int
    lib.mss_oracle_conv1d_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 4 + [ctypes.c_int, dp, dp]
    lib.mss_oracle_conv1d_fwd.restype = ctypes.c_int
    lib.mss_oracle_conv1d_update.argtypes = [i64, i64, i64, dp, dp, dp, dp, ctypes.c_int, dp]
    lib.mss_oracle_conv1d_update.restype = ctypes.c_int
    lib.mss_oracle_scan_fwd_complex.argtypes = [i64, i64, i64, i64] + [dp] * 10 + [
        ctypes.c_int, dp, dp, ctypes.c_int]
    lib.mss_oracle_scan_fwd_complex.restype = ctypes.c_int
    return lib


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library."""
    global _lib
    if path != LIB_PATH:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _f64(x, shape=None):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: exact upcast on the CPU
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def softplus(x: float, lib=None) -> float:
    return (lib or load()).mss_oracle_softplus(float(x))


def silu(x: float, lib=None) -> float:
    return (lib or load()).mss_oracle_silu(float(x))


def max_threads(lib=None) -> int:
    return (lib or load()).mss_oracle_max_threads()


def scan_fwd(u, delta_raw, A_log, B, C, D=None, z=None, dt_bias=None, h0=None,
             delta_softplus=True, threads=0, lib=None):
    """Selective-scan forward in fp64.  Returns (out [b,d,l], final_state [b,d,n])."""
    u = _f64(u)
    batch, dim, seqlen = u.shape
    A_log = _f64(A_log)
    dstate = A_log.shape[1]
    delta_raw = _f64(delta_raw, (batch, dim, seqlen))
    A_log = _f64(A_log, (dim, dstate))
    B = _f64(B, (batch, dstate, seqlen))
    C = _f64(C, (batch, dstate, seqlen))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, seqlen))
    dt_bias = _f64(dt_bias, (dim,))
    h0 = _f64(h0, (batch, dim, dstate))
    out = np.empty((batch, dim, seqlen), dtype=np.float64)
    final = np.empty((batch, dim, dstate), dtype=np.float64)
    rc = (lib or load()).mss_oracle_scan_fwd(
        batch, dim, seqlen, dstate, _ptr(u), _ptr(delta_raw), _ptr(A_log), _ptr(B),
        _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), int(bool(delta_softplus)),
        _ptr(out), _ptr(final), int(threads))
    if rc != 0:
        raise ValueError(f"oracle scan_fwd rejected its arguments (rc={rc})")
    return out, final


def _c128(x, shape=None):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: exact upcast on the CPU
        import torch
        x = x.detach().to("cpu", torch.complex128).numpy()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.complex128))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def scan_fwd_complex(u, delta_raw, A_log, A_imag, B, C, D=None, z=None, dt_bias=None, h0=None,
                     delta_softplus=True, threads=0, lib=None):
    """Selective-scan forward with complex A = -exp(A_log) + i A_imag, complex
    B, C and state, in fp64.  Returns (out [b,d,l] real, final_state [b,d,n]
    complex)."""
    u = _f64(u)
    batch, dim, seqlen = u.shape
    A_log = _f64(A_log)
    dstate = A_log.shape[1]
    delta_raw = _f64(delta_raw, (batch, dim, seqlen))
    A_imag = _f64(A_imag, (dim, dstate))
    B = _c128(B, (batch, dstate, seqlen))
    C = _c128(C, (batch, dstate, seqlen))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, seqlen))
    dt_bias = _f64(dt_bias, (dim,))
    h0 = _c128(h0, (batch, dim, dstate))
    out = np.empty((batch, dim, seqlen), dtype=np.float64)
    final = np.empty((batch, dim, dstate), dtype=np.complex128)
    rc = (lib or load()).mss_oracle_scan_fwd_complex(
        batch, dim, seqlen, dstate, _ptr(u), _ptr(delta_raw), _ptr(A_log), _ptr(A_imag),
        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), int(bool(delta_softplus)),
        _ptr(out), _ptr(final), int(threads))
    if rc != 0:
        raise ValueError(f"oracle scan_fwd_complex rejected its arguments (rc={rc})")
    return out, final


def state_update(state, u, delta_raw, A_log, B, C, D=None, z=None, dt_bias=None,
                 delta_softplus=True, lib=None):
    """One decode step in fp64.  Returns (out [b,d], new_state [b,d,n]); the
    input ``state`` is not modified."""
    new_state = _f64(state).copy()
    batch, dim, dstate = new_state.shape
    u = _f64(u, (batch, dim))
    delta_raw = _f64(delta_raw, (batch, dim))
    A_log = _f64(A_log, (dim, dstate))
    B = _f64(B, (batch, dstate))
    C = _f64(C, (batch, dstate))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim))
    dt_bias = _f64(dt_bias, (dim,))
    out = np.empty((batch, dim), dtype=np.float64)
    rc = (lib or load()).mss_oracle_state_update(
        batch, dim, dstate, _ptr(new_state), _ptr(u), _ptr(delta_raw), _ptr(A_log),
        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), int(bool(delta_softplus)),
        _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle state_update rejected its arguments (rc={rc})")
    return out, new_state


def scan_channels(inputs: dict, channels, delta_softplus=True, use_h0=False, threads=0):
    """Run the oracle on selected channels only.

    ``inputs`` holds arrays in logical index order (u [b,d,l], B [b,n,l], ...),
    any numpy/torch layout.  ``channels`` is a list of (b, d) pairs.  Returns
    (out [k, seqlen], final_state [k, dstate]) in the order given.
    """
    ch = list(channels)
    out = [None] * len(ch)
    fin = [None] * len(ch)
    by_b: dict[int, list[tuple[int, int]]] = {}
    for i, (b, d) in enumerate(ch):
        by_b.setdefault(int(b), []).append((i, int(d)))

    def pick(name, idx):
        x = inputs.get(name)
        if x is None:
            return None
        if hasattr(x, "detach"):
            import torch
            return x[idx].detach().to("cpu", torch.float64).numpy()
        return np.asarray(x[idx], dtype=np.float64)

    for b, items in by_b.items():
        ds = np.array([d for _, d in items], dtype=np.int64)
        sub = {
            "u": pick("u", (slice(b, b + 1), ds)),
            "delta_raw": pick("delta_raw", (slice(b, b + 1), ds)),
            "z": pick("z", (slice(b, b + 1), ds)),
            "B": pick("B", slice(b, b + 1)),
            "C": pick("C", slice(b, b + 1)),
            "A_log": pick("A_log", ds),
            "D": pick("D", ds),
            "dt_bias": pick("dt_bias", ds),
            "h0": pick("h0", (slice(b, b + 1), ds)) if use_h0 else None,
        }
        o, f = scan_fwd(sub["u"], sub["delta_raw"], sub["A_log"], sub["B"], sub["C"],
                        D=sub["D"], z=sub["z"], dt_bias=sub["dt_bias"], h0=sub["h0"],
                        delta_softplus=delta_softplus, threads=threads)
        for j, (i, _) in enumerate(items):
            out[i] = o[0, j]
            fin[i] = f[0, j]
    return np.stack(out), np.stack(fin)


def conv1d_fwd(x, w, bias=None, init=None, silu=True, lib=None):
    """Causal depthwise conv1d (+ SiLU) in fp64.

    x [b, d, l]; w [d, width]; bias [d]; init [b, d, width-1] (the carried
    window, oldest first; None means zeros).  Returns (out [b, d, l],
    final_window [b, d, width-1])."""
    x = _f64(x)
    batch, dim, seqlen = x.shape
    w = _f64(w)
    width = w.shape[1]
    w = _f64(w, (dim, width))
    bias = _f64(bias, (dim,))
    init = _f64(init, (batch, dim, width - 1))
    out = np.empty((batch, dim, seqlen), dtype=np.float64)
    final = np.empty((batch, dim, width - 1), dtype=np.float64)
    rc = (lib or load()).mss_oracle_conv1d_fwd(
        batch, dim, seqlen, width, _ptr(x), _ptr(w), _ptr(bias), _ptr(init), int(bool(silu)),
        _ptr(out), _ptr(final))
    if rc != 0:
        raise ValueError(f"oracle conv1d_fwd rejected its arguments (rc={rc})")
    return out, final


def conv1d_update(state, x, w, bias=None, silu=True, lib=None):
    """One conv1d decode step in fp64.  Returns (out [b, d], new_state
    [b, d, width-1]); the input ``state`` is not modified."""
    w = _f64(w)
    dim, width = w.shape
    x = _f64(x)
    batch = x.shape[0]
    x = _f64(x, (batch, dim))
    new_state = _f64(state, (batch, dim, width - 1)).copy()
    bias = _f64(bias, (dim,))
    out = np.empty((batch, dim), dtype=np.float64)
    rc = (lib or load()).mss_oracle_conv1d_update(
        batch, dim, width, _ptr(new_state), _ptr(x), _ptr(w), _ptr(bias), int(bool(silu)),
        _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle conv1d_update rejected its arguments (rc={rc})")
    return out, new_state


def scan_bwd(u, delta_raw, A_log, B, C, dout, D=None, z=None, dt_bias=None, h0=None,
             dfinal=None, delta_softplus=True, lib=None):
    """Backward of scan_fwd in fp64.

    Given dout [b,d,l] (and optionally dfinal [b,d,n], the gradient with respect
    to the exported final state), returns a dict of gradients: du, ddelta_raw
    [b,d,l]; dA_log [d,n]; dB, dC [b,n,l]; dD, ddt_bias [d] (always computed);
    dz [b,d,l] when z is given; dh0 [b,d,n]."""
    u = _f64(u)
    batch, dim, seqlen = u.shape
    A_log = _f64(A_log)
    dstate = A_log.shape[1]
    delta_raw = _f64(delta_raw, (batch, dim, seqlen))
    A_log = _f64(A_log, (dim, dstate))
    B = _f64(B, (batch, dstate, seqlen))
    C = _f64(C, (batch, dstate, seqlen))
    D = _f64(D, (dim,))
    z = _f64(z, (batch, dim, seqlen))
    dt_bias = _f64(dt_bias, (dim,))
    h0 = _f64(h0, (batch, dim, dstate))
    dout = _f64(dout, (batch, dim, seqlen))
    dfinal = _f64(dfinal, (batch, dim, dstate))
    g = {
        "du": np.empty((batch, dim, seqlen)), "ddelta_raw": np.empty((batch, dim, seqlen)),
        "dA_log": np.empty((dim, dstate)), "dB": np.empty((batch, dstate, seqlen)),
        "dC": np.empty((batch, dstate, seqlen)), "dD": np.empty(dim),
        "dz": np.empty((batch, dim, seqlen)) if z is not None else None,
        "ddt_bias": np.empty(dim), "dh0": np.empty((batch, dim, dstate)),
    }
    rc = (lib or load()).mss_oracle_scan_bwd(
        batch, dim, seqlen, dstate, _ptr(u), _ptr(delta_raw), _ptr(A_log), _ptr(B), _ptr(C),
        _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), int(bool(delta_softplus)), _ptr(dout),
        _ptr(dfinal), _ptr(g["du"]), _ptr(g["ddelta_raw"]), _ptr(g["dA_log"]), _ptr(g["dB"]),
        _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddt_bias"]), _ptr(g["dh0"]))
    if rc != 0:
        raise ValueError(f"oracle scan_bwd rejected its arguments (rc={rc})")
    return g
