"""Pins for the fp64 conv1d oracle: checks against things other than the oracle.

Each pin takes the oracle's ctypes library as an argument so that the same
checks run against deliberately broken copies of the oracle
(test_oracle_mutants.py).  A pin raises AssertionError when it fails.

What pins what:
  * the causal filter (zero left edge) -> scipy.signal.lfilter, the FIR filter
        y[t] = sum_j b[j] x[t - j]  with  b[j] = w[width - 1 - j]
    (a framework Conv1d is a cross-correlation, so its taps run oldest first)
  * a carried left window               -> numpy.convolve in 'valid' mode over
                                          the window followed by x
  * the activation                      -> 50-digit mpmath SiLU of the
                                          pre-activation
  * tap order and causality             -> the impulse response: a unit sample
                                          at t0 yields w[width-1-j] at t0+j
  * final window and carried window     -> a sequence cut anywhere and chained
                                          through the exported window equals
                                          the uncut run, bitwise
  * the decode step                     -> iterating it equals the full-sequence
                                          conv, bitwise
"""

from __future__ import annotations

import mpmath as mp
import numpy as np
from scipy.signal import lfilter

import oracle


def rand_conv(rng, batch, dim, L, width, *, with_bias=True, with_init=False):
    return {
        "x": rng.standard_normal((batch, dim, L)),
        "w": rng.standard_normal((dim, width)) * 0.5,
        "bias": rng.standard_normal(dim) * 0.3 if with_bias else None,
        "init": rng.standard_normal((batch, dim, width - 1)) if with_init else None,
    }


def _mp_silu(v):
    with mp.workdps(50):
        v = mp.mpf(float(v))
        return float(v / (1 + mp.exp(-v)))


def pin_conv_lfilter(lib):
    """Zero left edge: the pre-activation is bias + an FIR filter of x."""
    rng = np.random.default_rng(11)
    for width in (1, 2, 3, 4):
        for L in (1, 2, 3, 5, 40):
            for with_bias in (True, False):
                p = rand_conv(rng, 2, 3, L, width, with_bias=with_bias)
                pre, _ = oracle.conv1d_fwd(p["x"], p["w"], p["bias"], silu=False, lib=lib)
                for b in range(2):
                    for d in range(3):
                        ref = lfilter(p["w"][d, ::-1], [1.0], p["x"][b, d])
                        if with_bias:
                            ref = ref + p["bias"][d]
                        np.testing.assert_allclose(pre[b, d], ref, rtol=1e-13, atol=1e-13,
                                                   err_msg=f"width={width} L={L}")


def pin_conv_carried_window(lib):
    """A carried window: 'valid' convolution over the window followed by x."""
    rng = np.random.default_rng(12)
    for width in (2, 3, 4):
        for L in (1, 2, 7):
            p = rand_conv(rng, 1, 4, L, width, with_init=True)
            pre, _ = oracle.conv1d_fwd(p["x"], p["w"], p["bias"], p["init"], silu=False, lib=lib)
            for d in range(4):
                ext = np.concatenate([p["init"][0, d], p["x"][0, d]])
                ref = np.convolve(ext, p["w"][d, ::-1], mode="valid") + p["bias"][d]
                np.testing.assert_allclose(pre[0, d], ref, rtol=1e-13, atol=1e-13,
                                           err_msg=f"width={width} L={L}")


def pin_conv_silu(lib):
    """The activation is SiLU of the pre-activation, checked at 50 digits."""
    rng = np.random.default_rng(13)
    p = rand_conv(rng, 1, 3, 9, 4, with_init=True)
    p["x"] *= 4.0   # pre-activations over roughly [-8, 8]
    pre, _ = oracle.conv1d_fwd(p["x"], p["w"], p["bias"], p["init"], silu=False, lib=lib)
    out, _ = oracle.conv1d_fwd(p["x"], p["w"], p["bias"], p["init"], silu=True, lib=lib)
    ref = np.vectorize(_mp_silu)(pre)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-15)


def pin_conv_impulse(lib):
    """A unit sample at t0 yields w[width-1-j] at t0+j and 0 elsewhere."""
    for width in (1, 2, 3, 4):
        w = np.arange(1, width + 1, dtype=np.float64).reshape(1, width) * 0.25
        for t0 in (0, 2, 9):
            x = np.zeros((1, 1, 12))
            x[0, 0, t0] = 1.0
            pre, fin = oracle.conv1d_fwd(x, w, None, silu=False, lib=lib)
            ref = np.zeros(12)
            for j in range(width):
                if t0 + j < 12:
                    ref[t0 + j] = w[0, width - 1 - j]
            assert np.array_equal(pre[0, 0], ref), (width, t0, pre[0, 0], ref)


def pin_conv_chunked(lib):
    """Cut anywhere and chained through the exported window: bitwise equal."""
    rng = np.random.default_rng(14)
    for width in (1, 2, 4):
        for silu in (True, False):
            p = rand_conv(rng, 2, 3, 23, width, with_init=True)
            full, fin = oracle.conv1d_fwd(p["x"], p["w"], p["bias"], p["init"], silu=silu, lib=lib)
            for cuts in ((1,), (2, 3), (5, 6, 7, 20), (11,)):
                edges = [0, *cuts, 23]
                win = p["init"]
                parts = []
                for a, b in zip(edges[:-1], edges[1:]):
                    o, win = oracle.conv1d_fwd(p["x"][:, :, a:b], p["w"], p["bias"], win,
                                               silu=silu, lib=lib)
                    parts.append(o)
                assert np.array_equal(np.concatenate(parts, axis=2), full), (width, cuts)
                assert np.array_equal(win, fin), (width, cuts)


def pin_conv_step_equals_fwd(lib):
    """The separately written decode step, iterated, equals the full conv."""
    rng = np.random.default_rng(15)
    for width in (1, 2, 3, 4):
        for silu in (True, False):
            p = rand_conv(rng, 2, 5, 9, width, with_init=True)
            full, fin = oracle.conv1d_fwd(p["x"], p["w"], p["bias"], p["init"], silu=silu, lib=lib)
            state = p["init"]
            for t in range(9):
                y, state = oracle.conv1d_update(state, p["x"][:, :, t], p["w"], p["bias"],
                                                silu=silu, lib=lib)
                assert np.array_equal(y, full[:, :, t]), (width, silu, t)
            assert np.array_equal(state, fin), (width, silu)


ALL_CONV_PINS = [pin_conv_lfilter, pin_conv_carried_window, pin_conv_silu, pin_conv_impulse,
                 pin_conv_chunked, pin_conv_step_equals_fwd]
