"""Build libmss.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m mamba_selective_scan_amd.build   (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmss.so")
SOURCES = ["mss_api.hip", "scan_fwd.hip", "state_update.hip", "conv1d.hip", "scan_bwd.hip",
           "scan_cplx.hip"]
ARCH = "gfx950"

# Packed fp32 instructions are disabled for every kernel: the compiler would
# otherwise form them from ordinary float code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc, what, verbose):
    text, _ = proc.communicate()
    # hipcc's host pass does not know the packed-fp32 target feature and says
    # so; that message is expected and carries no information.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in text.splitlines() if noise not in ln and ln.strip()]
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({what}):\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)


def build(out: str = LIB_PATH, extra_flags=(), verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel, ``jobs`` at a time;
    0 = one per source up to the CPU count) and link libmss.so."""
    import tempfile
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="mss_build_") as tmpdir:
        objs, pending = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmd = [hipcc(), *compile_flags, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            pending.append((src, cmd))
        running = []
        while pending or running:
            while pending and len(running) < jobs:
                src, cmd = pending.pop(0)
                running.append((src, _run(cmd, verbose)))
            src, proc = running.pop(0)
            _finish(proc, src, verbose)
        tmp = out + ".tmp"
        link = [hipcc(), *HIP_FLAGS, *extra_flags, *objs, "-o", tmp]
        _finish(_run(link, verbose), "link", verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
