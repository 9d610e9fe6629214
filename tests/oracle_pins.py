"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes the oracle's ctypes library as an argument so that the same
checks can be run against deliberately broken copies of the oracle (see
test_oracle_mutants.py).  A pin raises AssertionError when it fails.

What pins what:
  * scalar softplus / silu            -> 50-digit mpmath evaluation of their
                                         textbook definitions on a grid
  * the recurrence and discretisation  -> the unrolled solution
        h_t = prod_{r<=t} a_r h_{-1} + sum_{s<=t} (prod_{s<r<=t} a_r) b_s,
        prod_r exp(Delta_r A) = exp(A sum_r Delta_r),
    evaluated in 50-digit mpmath for L <= 8, N in {1, 3}, every optional input
    present or absent, softplus on and off
  * long sequences                     -> the geometric-series closed form for
                                         inputs constant in time (L = 32768)
  * final state and initial state      -> composing segment aggregates with the
                                         pair operator (a2, b2) o (a1, b1) =
                                         (a2 a1, a2 b1 + b2), and chunked runs
                                         chained through the exported state
  * the state update                   -> iterating it equals the scan
  * special cases                      -> Delta = 0, B = 0, C = 0, a -> 0, L = 1
  * invariants                         -> linearity in u, causality (bitwise)
"""

from __future__ import annotations

import math
from fractions import Fraction

import mpmath as mp
import numpy as np

import oracle
from util import rel_err

DPS = 50


# ---------------------------------------------------------------- helpers ---

def rand_problem(rng, batch, dim, L, N, *, with_D=True, with_z=True, with_bias=True,
                 with_h0=False, delta_scale=0.5):
    p = {
        "u": rng.standard_normal((batch, dim, L)),
        "delta_raw": rng.standard_normal((batch, dim, L)) * delta_scale,
        "A_log": rng.standard_normal((dim, N)) * 0.5,
        "B": rng.standard_normal((batch, N, L)),
        "C": rng.standard_normal((batch, N, L)),
        "D": rng.standard_normal(dim) if with_D else None,
        "z": rng.standard_normal((batch, dim, L)) if with_z else None,
        "dt_bias": rng.standard_normal(dim) * 0.5 if with_bias else None,
        "h0": rng.standard_normal((batch, dim, N)) if with_h0 else None,
    }
    return p


def run_oracle(lib, p, softplus=True):
    return oracle.scan_fwd(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], D=p["D"],
                           z=p["z"], dt_bias=p["dt_bias"], h0=p.get("h0"),
                           delta_softplus=softplus, lib=lib)


def mp_softplus(x):
    return mp.log(1 + mp.exp(x))


def mp_silu(z):
    return z / (1 + mp.exp(-z))


def mp_unrolled(p, softplus=True):
    """50-digit evaluation of the unrolled recurrence solution (see module doc)."""
    u, dr, A_log = p["u"], p["delta_raw"], p["A_log"]
    Bm, Cm, D, z, bias, h0 = p["B"], p["C"], p["D"], p["z"], p["dt_bias"], p.get("h0")
    batch, dim, L = u.shape
    N = A_log.shape[1]
    out = np.zeros((batch, dim, L))
    fin = np.zeros((batch, dim, N))
    with mp.workdps(DPS):
        for b in range(batch):
            for d in range(dim):
                x = [mp.mpf(float(dr[b, d, t])) + (mp.mpf(float(bias[d])) if bias is not None else 0)
                     for t in range(L)]
                delta = [mp_softplus(v) if softplus else v for v in x]
                S = [mp.mpf(0)]
                for t in range(L):
                    S.append(S[-1] + delta[t])      # S[t+1] = sum_{r<=t} delta_r
                A = [-mp.exp(mp.mpf(float(A_log[d, n]))) for n in range(N)]
                for t in range(L):
                    y = mp.mpf(0)
                    for n in range(N):
                        h = mp.mpf(0)
                        if h0 is not None:
                            h += mp.exp(A[n] * S[t + 1]) * mp.mpf(float(h0[b, d, n]))
                        for s in range(t + 1):
                            bs = delta[s] * mp.mpf(float(Bm[b, n, s])) * mp.mpf(float(u[b, d, s]))
                            h += mp.exp(A[n] * (S[t + 1] - S[s + 1])) * bs
                        y += mp.mpf(float(Cm[b, n, t])) * h
                        if t == L - 1:
                            fin[b, d, n] = float(h)
                    if D is not None:
                        y += mp.mpf(float(D[d])) * mp.mpf(float(u[b, d, t]))
                    if z is not None:
                        y *= mp_silu(mp.mpf(float(z[b, d, t])))
                    out[b, d, t] = float(y)
    return out, fin


# ------------------------------------------------------------------- pins ---

def pin_scalars(lib):
    xs = list(np.linspace(-60, 60, 241)) + [0.0, 1e-300, -1e-8, 1e-8, 19.99, 20.01, -745.0, 700.0]
    with mp.workdps(DPS):
        for x in xs:
            ref = float(mp_softplus(mp.mpf(float(x))))
            got = oracle.softplus(x, lib=lib)
            assert abs(got - ref) <= 4e-16 * max(abs(ref), 1e-300), ("softplus", x, got, ref)
        for zv in list(np.linspace(-40, 40, 161)) + [0.0, 1e-9, -1e-9]:
            ref = float(mp_silu(mp.mpf(float(zv))))
            got = oracle.silu(zv, lib=lib)
            assert abs(got - ref) <= 4e-16 * max(abs(ref), 1e-300), ("silu", zv, got, ref)


def pin_brute_force(lib, combos=None, seed=0):
    rng = np.random.default_rng(seed)
    if combos is None:
        combos = [(sp, D, z, bias, h0) for sp in (True, False) for D in (True, False)
                  for z in (True, False) for bias in (True, False) for h0 in (True, False)]
    for (sp, wD, wz, wb, wh) in combos:
        for (L, N) in ((1, 1), (5, 3), (8, 1)):
            p = rand_problem(rng, 2, 2, L, N, with_D=wD, with_z=wz, with_bias=wb, with_h0=wh)
            out, fin = run_oracle(lib, p, softplus=sp)
            ref_out, ref_fin = mp_unrolled(p, softplus=sp)
            e1, e2 = rel_err(out, ref_out), rel_err(fin, ref_fin)
            assert e1 <= 1e-13 and e2 <= 1e-13, ("brute force", (sp, wD, wz, wb, wh, L, N), e1, e2)


def pin_geometric(lib, L=32768):
    """u, Delta, B, C, z constant in t: h_t = a^{t+1} h0 + b (1 - a^{t+1}) / (1 - a)."""
    batch, dim, N = 1, 2, 4
    A_log = np.array([[-1.0, 0.0, 0.7, 2.0], [0.3, -0.4, 1.1, 0.05]])
    uval = np.array([0.8, -1.3])
    drval = np.array([-2.0, 0.4])
    bias = np.array([0.25, -0.1])
    Bv = np.array([0.5, -1.0, 2.0, 0.25])
    Cv = np.array([1.5, 0.75, -0.5, 1.0])
    Dv = np.array([0.9, -0.2])
    zv = np.array([0.6, -1.7])
    h0 = np.array([[[0.3, -0.2, 1.0, 0.5], [2.0, 0.0, -1.0, 0.1]]])
    p = {
        "u": np.broadcast_to(uval[None, :, None], (batch, dim, L)).copy(),
        "delta_raw": np.broadcast_to(drval[None, :, None], (batch, dim, L)).copy(),
        "A_log": A_log, "B": np.broadcast_to(Bv[None, :, None], (batch, N, L)).copy(),
        "C": np.broadcast_to(Cv[None, :, None], (batch, N, L)).copy(), "D": Dv,
        "z": np.broadcast_to(zv[None, :, None], (batch, dim, L)).copy(), "dt_bias": bias,
        "h0": h0,
    }
    out, fin = run_oracle(lib, p, softplus=True)
    t = np.arange(L, dtype=np.float64)
    ref = np.zeros((batch, dim, L))
    ref_fin = np.zeros((batch, dim, N))
    for d in range(dim):
        x = drval[d] + bias[d]
        delta = max(x, 0.0) + math.log1p(math.exp(-abs(x)))      # softplus, stable form
        y = np.zeros(L)
        for n in range(N):
            lam = delta * -math.exp(A_log[d, n])                  # log a
            at1 = np.exp(lam * (t + 1))                           # a^{t+1}
            geo = -np.expm1(lam * (t + 1)) / -math.expm1(lam)     # (1 - a^{t+1}) / (1 - a)
            h = at1 * h0[0, d, n] + delta * Bv[n] * uval[d] * geo
            y += Cv[n] * h
            ref_fin[0, d, n] = h[-1]
        y += Dv[d] * uval[d]
        y *= zv[d] / (1.0 + math.exp(-zv[d]))
        ref[0, d] = y
    e1, e2 = rel_err(out, ref), rel_err(fin, ref_fin)
    assert e1 <= 1e-11 and e2 <= 1e-11, ("geometric", e1, e2)


def compose(second, first):
    """Pair operator: (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2)."""
    a2, b2 = second
    a1, b1 = first
    return a2 * a1, a2 * b1 + b2


def pin_chunk_composition(lib, seed=1):
    rng = np.random.default_rng(seed)
    L, N = 96, 3
    p = rand_problem(rng, 2, 3, L, N, with_h0=True)
    full_out, full_fin = run_oracle(lib, p)
    cuts = [0, 17, 40, 41, 96]
    # (i) chained through the exported state: bitwise equal to the full run.
    h = p["h0"]
    outs = []
    for s, e in zip(cuts[:-1], cuts[1:]):
        q = dict(p)
        for k in ("u", "delta_raw", "z", "B", "C"):
            q[k] = p[k][:, :, s:e]
        q["h0"] = h
        o, h = run_oracle(lib, q)
        outs.append(o)
    assert np.array_equal(np.concatenate(outs, axis=2), full_out), "chunked out != unchunked"
    assert np.array_equal(h, full_fin), "chunked final state != unchunked"
    # (ii) segment aggregates composed with the pair operator.
    agg = (np.ones_like(full_fin), np.zeros_like(full_fin))
    for s, e in zip(cuts[:-1], cuts[1:]):
        q = dict(p)
        for k in ("u", "delta_raw", "z", "B", "C"):
            q[k] = p[k][:, :, s:e]
        q["h0"] = None
        _, h_end = run_oracle(lib, q)                           # segment state from zero
        x = q["delta_raw"] + p["dt_bias"][None, :, None]
        delta = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
        sum_delta = np.array([[math.fsum(delta[b, d]) for d in range(delta.shape[1])]
                              for b in range(delta.shape[0])])
        prod_a = np.exp(sum_delta[:, :, None] * -np.exp(p["A_log"])[None, :, :])
        agg = compose((prod_a, h_end), agg)
    fin = agg[0] * p["h0"] + agg[1]
    e = rel_err(fin, full_fin)
    assert e <= 1e-13, ("aggregate composition", e)


def pin_step_equals_scan(lib, seed=2):
    rng = np.random.default_rng(seed)
    L, N = 40, 4
    for sp, wz, wD, wb in ((True, True, True, True), (False, False, False, False),
                           (True, False, True, False)):
        p = rand_problem(rng, 2, 3, L, N, with_D=wD, with_z=wz, with_bias=wb, with_h0=True)
        full_out, full_fin = run_oracle(lib, p, softplus=sp)
        state = p["h0"]
        steps = []
        for t in range(L):
            o, state = oracle.state_update(
                state, p["u"][:, :, t], p["delta_raw"][:, :, t], p["A_log"], p["B"][:, :, t],
                p["C"][:, :, t], D=p["D"], z=None if p["z"] is None else p["z"][:, :, t],
                dt_bias=p["dt_bias"], delta_softplus=sp, lib=lib)
            steps.append(o)
        e1 = rel_err(np.stack(steps, axis=2), full_out)
        e2 = rel_err(state, full_fin)
        assert e1 <= 1e-14 and e2 <= 1e-14, ("step != scan", sp, e1, e2)


def pin_special_cases(lib, seed=3):
    rng = np.random.default_rng(seed)
    L, N = 12, 3
    base = rand_problem(rng, 2, 3, L, N)
    silu = base["z"] / (1.0 + np.exp(-base["z"]))
    skip = base["D"][None, :, None] * base["u"]
    # Delta == 0 exactly (softplus off, delta_raw = -dt_bias): a = 1, b = 0.
    p = dict(base)
    p["dt_bias"] = np.array([0.5, -0.25, 1.0])
    p["delta_raw"] = np.broadcast_to(-p["dt_bias"][None, :, None], base["u"].shape).copy()
    out, fin = run_oracle(lib, p, softplus=False)
    assert rel_err(out, skip * silu) <= 1e-15, "Delta=0"
    assert np.all(fin == 0.0), "Delta=0 final state"
    # B == 0: state never leaves zero.
    p = dict(base)
    p["B"] = np.zeros_like(base["B"])
    out, fin = run_oracle(lib, p)
    assert rel_err(out, skip * silu) <= 1e-15 and np.all(fin == 0.0), "B=0"
    # C == 0: only the skip term reaches y.
    p = dict(base)
    p["C"] = np.zeros_like(base["C"])
    out, _ = run_oracle(lib, p)
    assert rel_err(out, skip * silu) <= 1e-15, "C=0"
    # a -> 0 (huge A_log): h_t = b_t, y = Delta u sum_n C_n B_n + D u.
    p = dict(base)
    p["A_log"] = np.full_like(base["A_log"], 60.0)
    out, fin = run_oracle(lib, p)
    x = p["delta_raw"] + p["dt_bias"][None, :, None]
    delta = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    cb = np.einsum("bnt,bnt->bt", p["C"], p["B"])
    ref = (delta * p["u"] * cb[:, None, :] + skip) * silu
    assert rel_err(out, ref) <= 1e-14, "a->0"
    ref_fin = delta[:, :, -1:] * p["u"][:, :, -1:] * p["B"][:, None, :, -1]
    assert rel_err(fin, ref_fin) <= 1e-14, "a->0 final"
    # L == 1 from a zero state: the same formula at t = 0.
    p = dict(base)
    for k in ("u", "delta_raw", "z", "B", "C"):
        p[k] = base[k][:, :, :1]
    out, _ = run_oracle(lib, p)
    x = p["delta_raw"] + p["dt_bias"][None, :, None]
    delta = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    cb = np.einsum("bnt,bnt->bt", p["C"], p["B"])
    zz = p["z"]
    ref = (delta * p["u"] * cb[:, None, :] + p["D"][None, :, None] * p["u"]) * zz / (1 + np.exp(-zz))
    assert rel_err(out, ref) <= 1e-14, "L=1"


def pin_invariants(lib, seed=4):
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, 2, 3, 50, 4, with_h0=False)
    out, fin = run_oracle(lib, p)
    q = dict(p)
    q["u"] = 2.0 * p["u"]
    out2, fin2 = run_oracle(lib, q)
    assert np.array_equal(out2, 2.0 * out) and np.array_equal(fin2, 2.0 * fin), "linearity in u"
    t0 = 23
    q = dict(p)
    for k in ("u", "delta_raw", "z", "B", "C"):
        q[k] = p[k].copy()
        q[k][:, :, t0] += 0.5
    out3, _ = run_oracle(lib, q)
    assert np.array_equal(out3[:, :, :t0], out[:, :, :t0]), "causality"
    assert not np.array_equal(out3[:, :, t0], out[:, :, t0]), "perturbation had no effect"


def pin_operator_associativity(seed=5):
    """The pair operator is associative (exact rational arithmetic)."""
    rng = np.random.default_rng(seed)

    def rnd():
        return Fraction(int(rng.integers(-50, 51)), int(rng.integers(1, 20)))
    for _ in range(200):
        x, y, w = [(rnd(), rnd()) for _ in range(3)]
        assert compose(compose(w, y), x) == compose(w, compose(y, x))


ALL_PINS = [pin_scalars, pin_brute_force, pin_geometric, pin_chunk_composition,
            pin_step_equals_scan, pin_special_cases, pin_invariants]
