"""Helpers for the GPU parity tests: device inputs, oracle references and the
comparison, with progress lines printed before each GPU step."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from util import TOL_BF16, TOL_F32, rel_err


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device():
    import torch
    return torch.device("cuda:0")


def sample_channels(batch, dim, k, seed=0):
    """k distinct (b, d) channels: the tile edges plus random ones."""
    rng = np.random.default_rng(seed)
    edges = {(0, 0), (batch - 1, dim - 1), (0, min(63, dim - 1)), (batch - 1, min(64, dim - 1)),
             (batch // 2, dim // 2)}
    picks = set(edges)
    while len(picks) < min(k, batch * dim):
        picks.add((int(rng.integers(batch)), int(rng.integers(dim))))
    return sorted(picks)


def run_gpu(mss, dev_inputs, *, with_z=True, with_D=True, with_bias=True, softplus=True,
            initial_state=None, final=True):
    res = mss.selective_scan_fwd(
        dev_inputs["u"], dev_inputs["delta_raw"], dev_inputs["A_log"], dev_inputs["B"],
        dev_inputs["C"], D=dev_inputs["D"] if with_D else None,
        z=dev_inputs["z"] if with_z else None,
        dt_bias=dev_inputs["dt_bias"] if with_bias else None, delta_softplus=softplus,
        initial_state=initial_state, return_final_state=final)
    return res


def oracle_full(dev_inputs, *, with_z=True, with_D=True, with_bias=True, softplus=True,
                initial_state=None):
    return oracle.scan_fwd(dev_inputs["u"], dev_inputs["delta_raw"], dev_inputs["A_log"],
                           dev_inputs["B"], dev_inputs["C"],
                           D=dev_inputs["D"] if with_D else None,
                           z=dev_inputs["z"] if with_z else None,
                           dt_bias=dev_inputs["dt_bias"] if with_bias else None,
                           h0=initial_state, delta_softplus=softplus)


def tol_for(io_dtype):
    return TOL_BF16 if io_dtype == "bf16" else TOL_F32


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def check(name, out, ref, tol):
    e = rel_err(out, ref)
    note(f"{name}: err={e:.3e} tol={tol:.0e}")
    assert e <= tol, f"{name}: error {e:.3e} exceeds {tol:.0e}"
    return e
