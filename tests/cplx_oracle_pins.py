"""Pins for the fp64 complex-A forward oracle: checks against things other
than the complex oracle itself.

Each pin takes the oracle's ctypes library so that the same checks run
against deliberately broken copies (test_oracle_mutants.py).  A pin raises
AssertionError when it fails.  What pins what:
  * A_imag = 0 with real B, C, h0 -> the real forward oracle (a separate
        function, itself pinned), output and final state
  * every term, tiny sizes -> the closed product form of the recurrence,
        h_t = prod_(r<=t) a_r h0 + sum_(s<=t) prod_(s<r<=t) a_r b_s, with
        a_r = cmath.exp(delta_r A) evaluated in Python, softplus off
  * constant inputs -> the geometric series b (1 - a^(t+1)) / (1 - a)
  * conjugating A's imaginary part, B, C and h0 leaves the output unchanged
        and conjugates the final state
  * no input (B = 0) -> |h_t| = |h0| exp(-exp(A_log) sum delta): the decay
        lives in the real part of A only
  * Re(A) ~ 0 and B = 0 -> a pure rotation of h0 by A_imag sum delta
  * linearity in u (no initial state)
"""

from __future__ import annotations

import cmath
import math

import numpy as np

import oracle


def _problem(rng, batch, dim, L, N, h0=True):
    return {
        "u": rng.standard_normal((batch, dim, L)),
        "delta_raw": rng.standard_normal((batch, dim, L)) * 0.5,
        "A_log": rng.standard_normal((dim, N)) * 0.5,
        "A_imag": rng.standard_normal((dim, N)) * 2.0,
        "B": rng.standard_normal((batch, N, L)) + 1j * rng.standard_normal((batch, N, L)),
        "C": rng.standard_normal((batch, N, L)) + 1j * rng.standard_normal((batch, N, L)),
        "D": rng.standard_normal(dim),
        "z": rng.standard_normal((batch, dim, L)),
        "dt_bias": rng.standard_normal(dim) * 0.5,
        "h0": (rng.standard_normal((batch, dim, N)) + 1j * rng.standard_normal((batch, dim, N))
               if h0 else None),
    }


def _run(lib, p, softplus=True, **override):
    q = dict(p, **override)
    return oracle.scan_fwd_complex(q["u"], q["delta_raw"], q["A_log"], q["A_imag"], q["B"],
                                   q["C"], D=q["D"], z=q["z"], dt_bias=q["dt_bias"], h0=q["h0"],
                                   delta_softplus=softplus, lib=lib)


def pin_cplx_real_reduction(lib):
    rng = np.random.default_rng(41)
    p = _problem(rng, 2, 3, 9, 4)
    p["A_imag"] = np.zeros_like(p["A_imag"])
    p["B"], p["C"] = p["B"].real.copy(), p["C"].real.copy()
    p["h0"] = p["h0"].real.copy()
    out, fin = _run(lib, p)
    r_out, r_fin = oracle.scan_fwd(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], D=p["D"],
                                   z=p["z"], dt_bias=p["dt_bias"], h0=p["h0"], lib=lib)
    assert np.allclose(out, r_out, rtol=1e-13, atol=1e-13)
    assert np.allclose(fin.real, r_fin, rtol=1e-13, atol=1e-13)
    assert np.all(fin.imag == 0.0)


def pin_cplx_product_form(lib):
    rng = np.random.default_rng(42)
    for _ in range(3):
        p = _problem(rng, 1, 2, 6, 2)
        p["delta_raw"] = np.abs(p["delta_raw"]) * 0.4
        p["dt_bias"] = np.abs(p["dt_bias"]) * 0.2
        out, fin = _run(lib, p, softplus=False)
        L = p["u"].shape[2]
        for d in range(2):
            delta = [p["delta_raw"][0, d, t] + p["dt_bias"][d] for t in range(L)]
            A = [complex(-math.exp(p["A_log"][d, n]), p["A_imag"][d, n]) for n in range(2)]
            for t in range(L):
                y = 0.0 + 0.0j
                for n in range(2):
                    a = [cmath.exp(delta[r] * A[n]) for r in range(L)]
                    h = complex(p["h0"][0, d, n])
                    for r in range(t + 1):
                        h *= a[r]
                    for s in range(t + 1):
                        prod = 1.0 + 0.0j
                        for r in range(s + 1, t + 1):
                            prod *= a[r]
                        h += prod * delta[s] * p["B"][0, n, s] * p["u"][0, d, s]
                    y += p["C"][0, n, t] * h
                    if t == L - 1:
                        assert abs(fin[0, d, n] - h) <= 1e-12 * max(1.0, abs(h))
                zt = p["z"][0, d, t]
                expect = (y.real + p["D"][d] * p["u"][0, d, t]) * zt / (1.0 + math.exp(-zt))
                assert abs(out[0, d, t] - expect) <= 1e-12 * max(1.0, abs(expect)), (d, t)


def pin_cplx_geometric(lib):
    # constant delta, u and B along t, h0 = 0: h_t = b (1 - a^(t+1)) / (1 - a)
    rng = np.random.default_rng(43)
    L, N = 40, 3
    p = _problem(rng, 1, 1, L, N, h0=False)
    p["delta_raw"] = np.full((1, 1, L), 0.3)
    p["dt_bias"] = np.zeros(1)
    p["u"] = np.full((1, 1, L), 1.7)
    b_n = rng.standard_normal(N) + 1j * rng.standard_normal(N)
    p["B"] = np.repeat(b_n[None, :, None], L, axis=2)
    p["C"] = np.repeat((rng.standard_normal(N) + 1j * rng.standard_normal(N))[None, :, None], L,
                       axis=2)
    p["z"] = None
    p["D"] = None
    out, fin = _run(lib, p, softplus=False)
    A = -np.exp(p["A_log"][0]) + 1j * p["A_imag"][0]
    a = np.exp(0.3 * A)
    b = 0.3 * 1.7 * b_n
    t = np.arange(L)[:, None]
    h = b[None, :] * (1.0 - a[None, :] ** (t + 1)) / (1.0 - a[None, :])
    y = (p["C"][0].T * h).sum(axis=1).real
    assert np.allclose(out[0, 0], y, rtol=1e-11, atol=1e-12)
    assert np.allclose(fin[0, 0], h[-1], rtol=1e-11, atol=1e-12)


def pin_cplx_conjugation(lib):
    rng = np.random.default_rng(44)
    p = _problem(rng, 2, 3, 11, 4)
    out, fin = _run(lib, p)
    out2, fin2 = _run(lib, p, A_imag=-p["A_imag"], B=p["B"].conj(), C=p["C"].conj(),
                      h0=p["h0"].conj())
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-12)
    assert np.allclose(fin.conj(), fin2, rtol=1e-12, atol=1e-12)


def pin_cplx_modulus(lib):
    rng = np.random.default_rng(45)
    p = _problem(rng, 2, 3, 13, 4)
    p["B"] = np.zeros_like(p["B"])
    _, fin = _run(lib, p)
    x = p["delta_raw"] + p["dt_bias"][None, :, None]
    delta = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    decay = np.exp(-np.exp(p["A_log"])[None] * delta.sum(axis=2)[:, :, None])
    assert np.allclose(np.abs(fin), np.abs(p["h0"]) * decay, rtol=1e-12, atol=1e-14)


def pin_cplx_rotation(lib):
    rng = np.random.default_rng(46)
    p = _problem(rng, 1, 2, 10, 3)
    p["A_log"] = np.full_like(p["A_log"], -60.0)  # Re(A) = -exp(-60), below fp64 resolution here
    p["B"] = np.zeros_like(p["B"])
    _, fin = _run(lib, p, softplus=False)
    delta = (p["delta_raw"] + p["dt_bias"][None, :, None]).sum(axis=2)
    expect = p["h0"] * np.exp(1j * p["A_imag"][None] * delta[:, :, None])
    assert np.allclose(fin, expect, rtol=1e-12, atol=1e-12)


def pin_cplx_linear_in_u(lib):
    rng = np.random.default_rng(47)
    p = _problem(rng, 2, 3, 10, 4, h0=False)
    out, fin = _run(lib, p)
    out3, fin3 = _run(lib, p, u=-2.5 * p["u"])
    assert np.allclose(out3, -2.5 * out, rtol=1e-12, atol=1e-12)
    assert np.allclose(fin3, -2.5 * fin, rtol=1e-12, atol=1e-12)


ALL_CPLX_PINS = [pin_cplx_real_reduction, pin_cplx_product_form, pin_cplx_geometric,
                 pin_cplx_conjugation, pin_cplx_modulus, pin_cplx_rotation, pin_cplx_linear_in_u]
