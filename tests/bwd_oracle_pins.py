"""Pins for the fp64 backward oracle: checks against things other than the
backward oracle itself.

Each pin takes the oracle's ctypes library so that the same checks run
against deliberately broken copies (test_oracle_mutants.py).  A pin raises
AssertionError when it fails.

The loss is J = sum(dout * out) + sum(dfinal * final_state), so the backward
returns dJ/d(input) for every input.  What pins what:
  * every gradient, element by element -> central finite differences of the
        forward oracle (a separate function, itself pinned) at fp64, on a tiny
        problem with every optional input present
  * every gradient, every flag combination -> directional finite differences
        along random directions
  * the hand-derived chain rule as a whole -> reverse-mode automatic
        differentiation (torch.autograd, float64, CPU) of the forward written
        as plain tensor operations
  * scale structure -> out and final_state are linear in u (no initial state),
        in B (out and final state), in C and in D (out), and affine in h0, so
        sum(du*u), sum(dB*B), sum(dC*C), sum(dD*D) and sum(dh0*h0) equal the
        matching parts of J exactly (Euler's identity for degree-1 maps)
  * dfinal and dh0 plumbing -> a sequence cut in two and chained (the second
        half's dh0 is the first half's dfinal) gives the uncut gradients
"""

from __future__ import annotations

import numpy as np

import oracle

INPUTS = ("u", "delta_raw", "A_log", "B", "C", "D", "z", "dt_bias", "h0")
GRAD_OF = {"u": "du", "delta_raw": "ddelta_raw", "A_log": "dA_log", "B": "dB", "C": "dC",
           "D": "dD", "z": "dz", "dt_bias": "ddt_bias", "h0": "dh0"}


def rand_bwd_problem(rng, batch, dim, L, N, *, with_D=True, with_z=True, with_bias=True,
                     with_h0=True, with_dfinal=True):
    return {
        "u": rng.standard_normal((batch, dim, L)),
        "delta_raw": rng.standard_normal((batch, dim, L)) * 0.5,
        "A_log": rng.standard_normal((dim, N)) * 0.5,
        "B": rng.standard_normal((batch, N, L)),
        "C": rng.standard_normal((batch, N, L)),
        "D": rng.standard_normal(dim) if with_D else None,
        "z": rng.standard_normal((batch, dim, L)) if with_z else None,
        "dt_bias": rng.standard_normal(dim) * 0.5 if with_bias else None,
        "h0": rng.standard_normal((batch, dim, N)) if with_h0 else None,
        "dout": rng.standard_normal((batch, dim, L)),
        "dfinal": rng.standard_normal((batch, dim, N)) if with_dfinal else None,
    }


def loss(lib, p, softplus=True, **override):
    q = dict(p, **override)
    out, fin = oracle.scan_fwd(q["u"], q["delta_raw"], q["A_log"], q["B"], q["C"], D=q["D"],
                               z=q["z"], dt_bias=q["dt_bias"], h0=q["h0"],
                               delta_softplus=softplus, lib=lib)
    j = float(np.sum(out * q["dout"]))
    if q["dfinal"] is not None:
        j += float(np.sum(fin * q["dfinal"]))
    return j


def grads(lib, p, softplus=True):
    return oracle.scan_bwd(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["dout"],
                           D=p["D"], z=p["z"], dt_bias=p["dt_bias"], h0=p["h0"],
                           dfinal=p["dfinal"], delta_softplus=softplus, lib=lib)


def pin_bwd_elementwise_fd(lib):
    """Every element of every gradient against a central difference."""
    rng = np.random.default_rng(31)
    eps = 1e-6
    for softplus in (True, False):
        p = rand_bwd_problem(rng, 2, 2, 4, 2)
        if not softplus:
            p["delta_raw"] = np.abs(p["delta_raw"]) * 0.3
        g = grads(lib, p, softplus)
        for name in INPUTS:
            x = p[name]
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                fd[idx] = (loss(lib, p, softplus, **{name: xp}) -
                           loss(lib, p, softplus, **{name: xm})) / (2 * eps)
            got = g[GRAD_OF[name]]
            scale = max(1.0, float(np.max(np.abs(fd))))
            assert np.max(np.abs(got - fd)) <= 1e-7 * scale, (name, softplus, got, fd)


def pin_bwd_directional_fd(lib):
    """Directional derivatives along random directions, every flag combination."""
    rng = np.random.default_rng(32)
    eps = 1e-6
    for softplus in (True, False):
        for with_D in (True, False):
            for with_z in (True, False):
                for with_bias in (True, False):
                    for with_h0 in (True, False):
                        p = rand_bwd_problem(rng, 2, 3, 6, 3, with_D=with_D, with_z=with_z,
                                             with_bias=with_bias, with_h0=with_h0,
                                             with_dfinal=with_h0)
                        if not softplus:
                            p["delta_raw"] = np.abs(p["delta_raw"]) * 0.3
                        g = grads(lib, p, softplus)
                        for name in INPUTS:
                            if p[name] is None:
                                continue
                            v = rng.standard_normal(p[name].shape)
                            fd = (loss(lib, p, softplus, **{name: p[name] + eps * v}) -
                                  loss(lib, p, softplus, **{name: p[name] - eps * v})) / (2 * eps)
                            got = float(np.sum(g[GRAD_OF[name]] * v))
                            scale = max(1.0, abs(fd))
                            assert abs(got - fd) <= 1e-7 * scale, (name, softplus, with_D, with_z,
                                                                   with_bias, with_h0, got, fd)


def pin_bwd_autograd(lib):
    """Reverse-mode autodiff of the forward written as plain tensor operations."""
    import torch
    rng = np.random.default_rng(33)
    for softplus in (True, False):
        p = rand_bwd_problem(rng, 2, 3, 7, 4)
        if not softplus:
            p["delta_raw"] = np.abs(p["delta_raw"]) * 0.3
        t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k in INPUTS)
             for k, v in p.items() if v is not None}
        A = -torch.exp(t["A_log"])
        x = t["delta_raw"] + t["dt_bias"][None, :, None]
        delta = (torch.clamp(x, min=0) + torch.log1p(torch.exp(-torch.abs(x)))) if softplus else x
        h = t["h0"]
        j = torch.zeros((), dtype=torch.float64)
        L = p["u"].shape[2]
        for s in range(L):
            a = torch.exp(delta[:, :, s, None] * A[None])
            h = a * h + delta[:, :, s, None] * t["B"][:, None, :, s] * t["u"][:, :, s, None]
            y = (h * t["C"][:, None, :, s]).sum(-1) + t["D"][None] * t["u"][:, :, s]
            zz = t["z"][:, :, s]
            j = j + (y * zz * torch.sigmoid(zz) * t["dout"][:, :, s]).sum()
        j = j + (h * t["dfinal"]).sum()
        j.backward()
        g = grads(lib, p, softplus)
        for name in INPUTS:
            ref = t[name].grad.numpy()
            assert np.allclose(g[GRAD_OF[name]], ref, rtol=1e-12, atol=1e-12), (name, softplus)


def pin_bwd_homogeneity(lib):
    """Euler's identity for the parts of J that are linear in one input."""
    rng = np.random.default_rng(34)
    p = rand_bwd_problem(rng, 2, 3, 9, 3, with_h0=False)
    g = grads(lib, p)
    out, fin = oracle.scan_fwd(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], D=p["D"],
                               z=p["z"], dt_bias=p["dt_bias"], lib=lib)
    gate = p["z"] / (1 + np.exp(-p["z"]))
    skip_part = float(np.sum(p["dout"] * p["D"][None, :, None] * p["u"] * gate))
    final_part = float(np.sum(fin * p["dfinal"]))
    j = float(np.sum(out * p["dout"])) + final_part
    ssm_out_part = j - skip_part - final_part
    tol = 1e-10 * max(1.0, abs(j))
    assert abs(float(np.sum(g["du"] * p["u"])) - j) <= tol
    assert abs(float(np.sum(g["dB"] * p["B"])) - (ssm_out_part + final_part)) <= tol
    assert abs(float(np.sum(g["dC"] * p["C"])) - ssm_out_part) <= tol
    assert abs(float(np.sum(g["dD"] * p["D"])) - skip_part) <= tol
    # affine in h0: J(h0) - J(0) = sum(dh0 * h0)
    q = rand_bwd_problem(rng, 2, 3, 9, 3, with_h0=True)
    gq = grads(lib, q)
    diff = loss(lib, q) - loss(lib, q, h0=None)
    assert abs(float(np.sum(gq["dh0"] * q["h0"])) - diff) <= 1e-10 * max(1.0, abs(diff))


def pin_bwd_chained_halves(lib):
    """Cut the sequence in two: forward the first half for its final state, run
    the second half's backward from it, feed its dh0 as the first half's
    dfinal.  The two halves' gradients equal the uncut ones."""
    rng = np.random.default_rng(35)
    p = rand_bwd_problem(rng, 2, 3, 11, 3)
    full = grads(lib, p)
    cut = 5
    first = {k: (v[:, :, :cut] if k in ("u", "delta_raw", "B", "C", "z", "dout") else v)
             for k, v in p.items()}
    second = {k: (v[:, :, cut:] if k in ("u", "delta_raw", "B", "C", "z", "dout") else v)
              for k, v in p.items()}
    _, mid = oracle.scan_fwd(first["u"], first["delta_raw"], first["A_log"], first["B"],
                             first["C"], D=first["D"], z=first["z"], dt_bias=first["dt_bias"],
                             h0=first["h0"], lib=lib)
    second["h0"] = mid
    g2 = grads(lib, second)
    first["dfinal"] = g2["dh0"]
    g1 = grads(lib, first)
    for k in ("du", "ddelta_raw", "dB", "dC", "dz"):
        joined = np.concatenate([g1[k], g2[k]], axis=2)
        assert np.allclose(joined, full[k], rtol=1e-12, atol=1e-12), k
    for k in ("dA_log", "dD", "ddt_bias"):
        assert np.allclose(g1[k] + g2[k], full[k], rtol=1e-12, atol=1e-12), k
    assert np.allclose(g1["dh0"], full["dh0"], rtol=1e-12, atol=1e-12)


ALL_BWD_PINS = [pin_bwd_elementwise_fd, pin_bwd_directional_fd, pin_bwd_autograd,
                pin_bwd_homogeneity, pin_bwd_chained_halves]
