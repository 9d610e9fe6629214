"""Shared test helpers: the error metric and small array utilities."""

from __future__ import annotations

import numpy as np

# Tolerances on the error metric below: fp32 I/O, and bf16 I/O with fp32 state.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def rel_err(out, ref) -> float:
    """max_i |o_i - r_i| / (|r_i| + rms(r)).

    A plain per-element relative error is unusable here: the output crosses
    zero (y * silu(z) changes sign), so a correct result can show an arbitrary
    element-wise relative error next to a zero.  Scaling by |r_i| + rms(r)
    keeps the element-wise character for large values and turns into an
    absolute error relative to the tensor's typical size near zero.  Complex
    arrays use complex moduli throughout (|o_i - r_i|, |r_i|, rms of |r|).
    """
    cplx = np.iscomplexobj(out) or np.iscomplexobj(ref)
    dt = np.complex128 if cplx else np.float64
    o = np.asarray(out, dtype=dt)
    r = np.asarray(ref, dtype=dt)
    if o.shape != r.shape:
        raise ValueError(f"shape mismatch {o.shape} vs {r.shape}")
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(np.abs(r) ** 2)))
    denom = np.abs(r) + rms
    if rms == 0.0:
        return float(np.max(np.abs(o - r)))
    return float(np.max(np.abs(o - r) / denom))


def l2_rel(out, ref) -> float:
    o = np.asarray(out, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    n = float(np.linalg.norm(r))
    return float(np.linalg.norm(o - r)) / (n if n > 0 else 1.0)
