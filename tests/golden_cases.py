"""Loader for the hand-derived worked examples in tests/golden/.

Each scan fixture lists its inputs and its expected outputs as exact rationals
c0 + c1 * ln(2); each conv fixture lists exact rationals.  See the header of each file for the derivation.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok: str) -> float:
    tok = tok.strip()
    if tok == "ln2":
        return math.log(2.0)
    return float(Fraction(tok))


def load(name: str) -> dict:
    fields = {}
    with open(os.path.join(GOLDEN_DIR, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            fields[k] = v
    kind = fields["kind"]
    vec = lambda k: np.array([_num(t) for t in fields[k].split(",")])
    if kind in ("conv", "conv_step"):
        w = vec("w")
        width = w.size
        case = {"kind": kind, "name": name, "w": w.reshape(1, width), "bias": vec("bias"),
                "final": vec("final").reshape(1, 1, width - 1)}
        if kind == "conv":
            x = vec("x")
            case["x"] = x.reshape(1, 1, x.size)
            case["y"] = vec("y").reshape(1, 1, x.size)
        else:
            case["state"] = vec("state").reshape(1, 1, width - 1)
            case["x"] = vec("x").reshape(1, 1)
            case["y"] = vec("y").reshape(1, 1)
        return case
    N = int(fields["dstate"])
    ln2 = math.log(2.0)
    case = {"kind": kind, "dstate": N, "name": name}
    if kind == "scan":
        L = int(fields["seqlen"])
        full = lambda v: np.full((1, 1, L), float(v[0]))
        case["u"] = full(vec("u"))
        case["delta_raw"] = full(vec("delta_raw"))
        case["A_log"] = vec("A_log").reshape(1, N)
        case["B"] = np.broadcast_to(vec("B").reshape(1, N, 1), (1, N, L)).copy()
        case["C"] = np.broadcast_to(vec("C").reshape(1, N, 1), (1, N, L)).copy()
        case["D"] = vec("D")
        case["y"] = (vec("y_const") + vec("y_ln2") * ln2).reshape(1, 1, L)
        case["final"] = (vec("final_const") + vec("final_ln2") * ln2).reshape(1, 1, N)
    else:
        case["state"] = vec("state").reshape(1, 1, N)
        case["u"] = vec("u").reshape(1, 1)
        case["delta_raw"] = vec("delta_raw").reshape(1, 1)
        case["A_log"] = vec("A_log").reshape(1, N)
        case["B"] = vec("B").reshape(1, N)
        case["C"] = vec("C").reshape(1, N)
        case["D"] = vec("D")
        case["y"] = (vec("y_const") + vec("y_ln2") * ln2).reshape(1, 1)
        case["final"] = (vec("final_const") + vec("final_ln2") * ln2).reshape(1, 1, N)
    return case


ALL = sorted(f for f in os.listdir(GOLDEN_DIR) if f.endswith(".txt"))
