"""The C ABI: every declared symbol is exported, the ctypes structs match the C
layout, and every argument check fires before any HIP call.

The argument-check tests pass fake device addresses; libmss rejects each call
on the host before touching them.  They are skipped on machines with a GPU
device node, so that a broken check could never launch on fake pointers.
"""

import ctypes
import os
import re
import subprocess

import pytest

from mamba_selective_scan_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mss.h")
HAS_GPU_NODE = os.path.exists("/dev/kfd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mss_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = _lib.lib()
    decl = declared_functions()
    assert set(decl) == set(_lib.EXPORTS), decl
    for name in decl:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mss_\w+)", out))
    assert set(decl) <= exported


def test_abi_version_and_status_strings():
    lib = _lib.lib()
    assert lib.mss_abi_version() == _lib.MSS_ABI_VERSION
    for code in _lib.STATUS:
        s = lib.mss_status_string(code)
        assert s and isinstance(s, bytes)
    assert lib.mss_status_string(999) == b"unknown status"


def _c_layout(struct_name, fields, tmp_path):
    src = tmp_path / "probe.c"
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "mss.h"', "int main(void){",
             f'printf("%zu\\n", sizeof({struct_name}));']
    for f in fields:
        lines.append(f'printf("%zu\\n", offsetof({struct_name}, {f}));')
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("cls,cname", [(_lib.ScanArgs, "mss_scan_args"),
                                       (_lib.StepArgs, "mss_step_args"),
                                       (_lib.ConvArgs, "mss_conv_args"),
                                       (_lib.ConvStepArgs, "mss_conv_step_args"),
                                       (_lib.ScanBwdArgs, "mss_scan_bwd_args"),
                                       (_lib.ScanComplexArgs, "mss_scan_complex_args")])
def test_ctypes_struct_matches_c_layout(cls, cname, tmp_path):
    names = [f[0] for f in cls._fields_]
    size, offs = _c_layout(cname, names, tmp_path)
    assert ctypes.sizeof(cls) == size
    assert [getattr(cls, n).offset for n in names] == offs


def test_workspace_size_depends_on_shape_only():
    lib = _lib.lib()
    a = _lib.new_scan_args()
    a.batch, a.dim, a.seqlen, a.dstate = 8, 5120, 4096, 16
    st = ctypes.c_int(-1)
    n = lib.mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
    assert st.value == 0
    assert n == 0                        # enough channel tiles: no time split, no scratch
    a.batch, a.dim, a.seqlen = 1, 256, 220500
    n2 = lib.mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
    assert st.value == 0 and n2 > 0      # few channels, long sequence: segment carries
    a.dstate = 17
    assert lib.mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st)) == 0
    assert st.value == _lib.STATUS_CODE["MSS_ERR_UNSUPPORTED_DSTATE"]
    assert lib.mss_selective_scan_workspace_size(None, ctypes.byref(st)) == 0
    assert st.value == _lib.STATUS_CODE["MSS_ERR_BAD_STRUCT"]


@pytest.mark.parametrize("dim,seqlen,parts", [(8192, 1117, 2), (1536, 2048, 1), (256, 220500, 2),
                                               (1536, 32768, 2)])
def test_scan_workspace_holds_aggregate_parts(dim, seqlen, parts):
    # Workspace = (nseg - 1) * parts aggregates (P, H) per padded channel and
    # state, nseg carries, and a state hand-off when the length is not a
    # multiple of 4.  The plan: segments fill 4096 waves of 8 channels; the
    # aggregate pass cuts each into `parts` (at most 2) while its grid, in whole
    # 32-channel blocks, stays at or below 8192 waves with parts of >= 4 chunks.
    lib = _lib.lib()
    a = _lib.new_scan_args()
    a.batch, a.dim, a.seqlen, a.dstate = 1, dim, seqlen, 16
    st = ctypes.c_int(-1)
    n = lib.mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
    assert st.value == 0
    tiles = (dim + 7) // 8
    chunks = (seqlen + 31) // 32
    nseg0 = max(1, min(4096 // tiles, chunks))
    seg_chunks = -(-chunks // nseg0)
    nseg = -(-seqlen // (seg_chunks * 32))
    blocks = -(-tiles // 4) * 4 * (nseg - 1)
    assert min(8192 // blocks, seg_chunks // 4, 2) == parts
    pad = tiles * 8
    up = lambda x: -(-x // 256) * 256
    want = up((nseg - 1) * parts * pad * 16 * 8) + up(nseg * pad * 16 * 4)
    if seqlen % 4:
        want += up(dim * 16 * 4)
    assert n == want


# ----------------------------------------------------------- argument checks

BASE = 0x7F0000000000
GAP = 1 << 32


def fake(i):
    return BASE + i * GAP


def scan_args(batch=2, dim=96, seqlen=100, dstate=16, ws=True):
    # this shape is split in time, so it needs a workspace: a call built with
    # ws=False stops at the workspace check at the latest
    a = _lib.new_scan_args()
    a.io_dtype = _lib.MSS_F32
    a.batch, a.dim, a.seqlen, a.dstate = batch, dim, seqlen, dstate
    x = (dim * seqlen, seqlen, 1)
    bc = (dstate * seqlen, seqlen, 1)
    a.u, a.u_stride = fake(0), (ctypes.c_int64 * 3)(*x)
    a.delta_raw, a.delta_stride = fake(1), (ctypes.c_int64 * 3)(*x)
    a.A_log, a.A_log_stride = fake(2), (ctypes.c_int64 * 2)(dstate, 1)
    a.B, a.B_stride = fake(3), (ctypes.c_int64 * 3)(*bc)
    a.C, a.C_stride = fake(4), (ctypes.c_int64 * 3)(*bc)
    a.D = fake(5)
    a.z, a.z_stride = fake(6), (ctypes.c_int64 * 3)(*x)
    a.dt_bias = fake(7)
    a.out, a.out_stride = fake(8), (ctypes.c_int64 * 3)(*x)
    a.final_state = fake(9)
    a.delta_softplus = 1
    if ws:
        st = ctypes.c_int(0)
        a.workspace = fake(10)
        a.workspace_bytes = _lib.lib().mss_selective_scan_workspace_size(ctypes.byref(a),
                                                                         ctypes.byref(st))
    return a


def code(name):
    return _lib.STATUS_CODE[name]


def call_scan(a):
    return _lib.lib().mss_selective_scan_fwd(ctypes.byref(a) if a is not None else None, None)


def _mut_scan(fn, ws=False):
    a = scan_args(ws=ws)
    fn(a)
    return a


SCAN_CASES = {
    "null_struct": (None, "MSS_ERR_BAD_STRUCT"),
    "struct_size": (lambda a: setattr(a, "struct_size", 8), "MSS_ERR_BAD_STRUCT"),
    "reverse2": (lambda a: setattr(a, "reverse", 2), "MSS_ERR_BAD_STRUCT"),
    "dtype": (lambda a: setattr(a, "io_dtype", 7), "MSS_ERR_UNSUPPORTED_DTYPE"),
    "batch0": (lambda a: setattr(a, "batch", 0), "MSS_ERR_BAD_SHAPE"),
    "seqlen_neg": (lambda a: setattr(a, "seqlen", -3), "MSS_ERR_BAD_SHAPE"),
    "seqlen_huge": (lambda a: setattr(a, "seqlen", 1 << 31), "MSS_ERR_BAD_SHAPE"),
    "dstate0": (lambda a: setattr(a, "dstate", 0), "MSS_ERR_UNSUPPORTED_DSTATE"),
    "dstate17": (lambda a: setattr(a, "dstate", 17), "MSS_ERR_UNSUPPORTED_DSTATE"),
    "u_null": (lambda a: setattr(a, "u", None), "MSS_ERR_NULL_POINTER"),
    "C_null": (lambda a: setattr(a, "C", None), "MSS_ERR_NULL_POINTER"),
    "out_null": (lambda a: setattr(a, "out", None), "MSS_ERR_NULL_POINTER"),
    "neg_stride": (lambda a: a.u_stride.__setitem__(1, -1), "MSS_ERR_BAD_STRIDE"),
    "out_overlap": (lambda a: a.out_stride.__setitem__(1, 0), "MSS_ERR_BAD_STRIDE"),
    "tile_2gib": (lambda a: a.u_stride.__setitem__(1, 1 << 27), "MSS_ERR_BAD_STRIDE"),
    "misaligned_u": (lambda a: setattr(a, "u", fake(0) + 2), "MSS_ERR_MISALIGNED"),
    # bf16 elements must be 2-byte aligned (a 4-byte misaligned bf16 view is
    # legal and runs the element-wise instantiation; see the GPU parity tests)
    "misaligned_bf16": (lambda a: (setattr(a, "io_dtype", _lib.MSS_BF16),
                                   setattr(a, "B", fake(3) + 1)), "MSS_ERR_MISALIGNED"),
    "misaligned_final": (lambda a: setattr(a, "final_state", fake(9) + 1), "MSS_ERR_MISALIGNED"),
    "out_is_u": (lambda a: setattr(a, "out", fake(0)), "MSS_ERR_ALIASING"),
    "final_in_z": (lambda a: setattr(a, "final_state", fake(6) + 64), "MSS_ERR_ALIASING"),
    "out_on_A_log": (lambda a: setattr(a, "out", fake(2) - 8), "MSS_ERR_ALIASING"),
    "misaligned_chunk_states": (lambda a: setattr(a, "chunk_states", fake(11) + 4),
                                "MSS_ERR_MISALIGNED"),
    "chunk_states_on_out": (lambda a: setattr(a, "chunk_states", fake(8) + 256), "MSS_ERR_ALIASING"),
    "chunk_states_on_u": (lambda a: setattr(a, "chunk_states", fake(0) - 8), "MSS_ERR_ALIASING"),
    "no_workspace": (lambda a: None, "MSS_ERR_WORKSPACE_TOO_SMALL"),
}


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(SCAN_CASES))
def test_scan_argument_checks(case):
    assert scan_args(ws=True).workspace_bytes > 0
    fn, expect = SCAN_CASES[case]
    a = None if fn is None else _mut_scan(fn)
    assert call_scan(a) == code(expect)


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
def test_scan_bc_layout_checks():
    """B and C need a shared unit-stride axis (t or n) unless both are
    time-invariant (time stride 0), which takes any state stride."""
    a = scan_args(ws=True)
    a.B_stride[2] = a.C_stride[2] = 3
    assert call_scan(a) == code("MSS_ERR_BAD_STRIDE")
    a = scan_args(ws=True)
    a.B_stride[2] = 0  # B time-invariant with state stride seqlen, C per step
    assert call_scan(a) == code("MSS_ERR_BAD_STRIDE")
    a = scan_args(ws=True)
    a.B_stride[2] = a.C_stride[2] = 0  # both time-invariant, state stride seqlen
    # every argument check passes; only the launch fails (no device here)
    assert call_scan(a) == code("MSS_ERR_HIP")


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
def test_scan_workspace_checks():
    a = scan_args(ws=True)
    a.workspace_bytes -= 1
    assert call_scan(a) == code("MSS_ERR_WORKSPACE_TOO_SMALL")
    a = scan_args(ws=True)
    a.workspace = fake(10) + 128
    assert call_scan(a) == code("MSS_ERR_MISALIGNED")
    a = scan_args(ws=True)
    a.workspace = fake(0)
    assert call_scan(a) == code("MSS_ERR_ALIASING")


def call_scan_noalloc(a):
    return _lib.lib().mss_selective_scan_fwd_noalloc(ctypes.byref(a) if a is not None else None,
                                                     None)


NOALLOC_CASES = {k: v for k, v in SCAN_CASES.items() if k != "no_workspace"}


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(NOALLOC_CASES))
def test_scan_noalloc_argument_checks(case):
    """The no-allocation forward runs every check of the forward, before any
    HIP call (including the scratch-address lookup)."""
    fn, expect = NOALLOC_CASES[case]
    a = None if fn is None else _mut_scan(fn)
    assert call_scan_noalloc(a) == code(expect)


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
def test_scan_noalloc_workspace_and_scratch_limit():
    # a workspace passed to the no-allocation entry point is a usage error
    a = scan_args(ws=True)
    assert call_scan_noalloc(a) == code("MSS_ERR_BAD_STRUCT")
    a = scan_args(ws=False)
    a.workspace_bytes = 64
    assert call_scan_noalloc(a) == code("MSS_ERR_BAD_STRUCT")
    # a ragged length over more channels than the scratch holds a state
    # hand-off for: rejected before any HIP call
    dim = _lib.MSS_NOALLOC_SCRATCH_BYTES // (16 * 4) + 8
    a = scan_args(batch=1, dim=dim, seqlen=3, ws=False)
    st = ctypes.c_int(-1)
    need = _lib.lib().mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
    assert st.value == 0 and need > _lib.MSS_NOALLOC_SCRATCH_BYTES
    assert call_scan_noalloc(a) == code("MSS_ERR_SCRATCH_LIMIT")


def test_noalloc_scratch_covers_every_segmented_shape():
    """Time segments are planned only below 2048 channel tiles (16384
    channels): their carries, plus a ragged-tail hand-off, fit the scratch for
    every such shape (the worst cases of the segment count are swept)."""
    lib = _lib.lib()
    st = ctypes.c_int(-1)
    worst = 0
    for channels in (8, 64, 256, 1024, 1536, 4096, 16376):
        for seqlen in (3, 4097, 65539, 1 << 20, (1 << 30) - 1):
            a = _lib.new_scan_args()
            a.batch, a.dim, a.seqlen, a.dstate = 1, channels, seqlen, 16
            n = lib.mss_selective_scan_workspace_size(ctypes.byref(a), ctypes.byref(st))
            assert st.value == 0
            worst = max(worst, n)
    assert 0 < worst <= _lib.MSS_NOALLOC_SCRATCH_BYTES


def step_args():
    a = _lib.new_step_args()
    a.io_dtype = _lib.MSS_F32
    a.batch, a.dim, a.dstate = 2, 96, 16
    x = (96, 1)
    a.state = fake(0)
    a.u, a.u_stride = fake(1), (ctypes.c_int64 * 2)(*x)
    a.delta_raw, a.delta_stride = fake(2), (ctypes.c_int64 * 2)(*x)
    a.A_log, a.A_log_stride = fake(3), (ctypes.c_int64 * 2)(16, 1)
    a.B, a.B_stride = fake(4), (ctypes.c_int64 * 2)(16, 1)
    a.C, a.C_stride = fake(5), (ctypes.c_int64 * 2)(16, 1)
    a.D = fake(6)
    a.z, a.z_stride = fake(7), (ctypes.c_int64 * 2)(*x)
    a.dt_bias = fake(8)
    a.out, a.out_stride = fake(9), (ctypes.c_int64 * 2)(*x)
    a.delta_softplus = 1
    return a


STEP_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), "MSS_ERR_BAD_STRUCT"),
    "dtype": (lambda a: setattr(a, "io_dtype", 2), "MSS_ERR_UNSUPPORTED_DTYPE"),
    "dim0": (lambda a: setattr(a, "dim", 0), "MSS_ERR_BAD_SHAPE"),
    "dstate20": (lambda a: setattr(a, "dstate", 20), "MSS_ERR_UNSUPPORTED_DSTATE"),
    "state_null": (lambda a: setattr(a, "state", None), "MSS_ERR_NULL_POINTER"),
    "neg_stride": (lambda a: a.B_stride.__setitem__(1, -1), "MSS_ERR_BAD_STRIDE"),
    "out_overlap": (lambda a: a.out_stride.__setitem__(1, 0), "MSS_ERR_BAD_STRIDE"),
    "misaligned": (lambda a: setattr(a, "state", fake(0) + 2), "MSS_ERR_MISALIGNED"),
    "out_is_u": (lambda a: setattr(a, "out", fake(1)), "MSS_ERR_ALIASING"),
    "state_on_B": (lambda a: setattr(a, "state", fake(4)), "MSS_ERR_ALIASING"),
}


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(STEP_CASES))
def test_step_argument_checks(case):
    fn, expect = STEP_CASES[case]
    a = step_args()
    fn(a)
    assert _lib.lib().mss_selective_state_update(ctypes.byref(a), None) == code(expect)


def conv_args(width=4):
    a = _lib.new_conv_args()
    a.io_dtype = _lib.MSS_F32
    a.batch, a.dim, a.seqlen, a.width = 2, 96, 100, width
    x = (96 * 100, 1, 96)             # channel-last [B, L, D] storage
    a.x, a.x_stride = fake(0), (ctypes.c_int64 * 3)(*x)
    a.weight, a.weight_stride = fake(1), (ctypes.c_int64 * 2)(width, 1)
    a.bias = fake(2)
    a.initial_state = fake(3)
    a.out, a.out_stride = fake(4), (ctypes.c_int64 * 3)(*x)
    a.final_state = fake(5)
    a.activation = _lib.MSS_ACT_SILU
    return a


CONV_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 12), "MSS_ERR_BAD_STRUCT"),
    "reserved": (lambda a: setattr(a, "reserved0", 3), "MSS_ERR_BAD_STRUCT"),
    "activation": (lambda a: setattr(a, "activation", 5), "MSS_ERR_BAD_STRUCT"),
    "dtype": (lambda a: setattr(a, "io_dtype", 9), "MSS_ERR_UNSUPPORTED_DTYPE"),
    "width0": (lambda a: setattr(a, "width", 0), "MSS_ERR_BAD_SHAPE"),
    "width5": (lambda a: setattr(a, "width", 5), "MSS_ERR_BAD_SHAPE"),
    "seqlen0": (lambda a: setattr(a, "seqlen", 0), "MSS_ERR_BAD_SHAPE"),
    "dim_huge": (lambda a: setattr(a, "dim", 1 << 31), "MSS_ERR_BAD_SHAPE"),
    "x_null": (lambda a: setattr(a, "x", None), "MSS_ERR_NULL_POINTER"),
    "weight_null": (lambda a: setattr(a, "weight", None), "MSS_ERR_NULL_POINTER"),
    "out_null": (lambda a: setattr(a, "out", None), "MSS_ERR_NULL_POINTER"),
    "neg_stride": (lambda a: a.x_stride.__setitem__(2, -96), "MSS_ERR_BAD_STRIDE"),
    "neg_weight_stride": (lambda a: a.weight_stride.__setitem__(0, -4), "MSS_ERR_BAD_STRIDE"),
    "out_overlap": (lambda a: a.out_stride.__setitem__(2, 0), "MSS_ERR_BAD_STRIDE"),
    "misaligned_x": (lambda a: setattr(a, "x", fake(0) + 2), "MSS_ERR_MISALIGNED"),
    "misaligned_bias": (lambda a: setattr(a, "bias", fake(2) + 1), "MSS_ERR_MISALIGNED"),
    "out_is_x": (lambda a: setattr(a, "out", fake(0)), "MSS_ERR_ALIASING"),
    "final_on_weight": (lambda a: setattr(a, "final_state", fake(1)), "MSS_ERR_ALIASING"),
    "final_in_out": (lambda a: setattr(a, "final_state", fake(4) + 400), "MSS_ERR_ALIASING"),
    "out_on_init": (lambda a: setattr(a, "out", fake(3) - 16), "MSS_ERR_ALIASING"),
}


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(CONV_CASES))
def test_conv_argument_checks(case):
    fn, expect = CONV_CASES[case]
    a = conv_args()
    fn(a)
    assert _lib.lib().mss_causal_conv1d_fwd(ctypes.byref(a), None) == code(expect)


def conv_step_args(width=4):
    a = _lib.new_conv_step_args()
    a.io_dtype = _lib.MSS_BF16
    a.batch, a.dim, a.width = 2, 96, width
    a.state = fake(0)
    a.x, a.x_stride = fake(1), (ctypes.c_int64 * 2)(96, 1)
    a.weight, a.weight_stride = fake(2), (ctypes.c_int64 * 2)(width, 1)
    a.bias = fake(3)
    a.out, a.out_stride = fake(4), (ctypes.c_int64 * 2)(96, 1)
    a.activation = _lib.MSS_ACT_NONE
    return a


CONV_STEP_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 0), "MSS_ERR_BAD_STRUCT"),
    "activation": (lambda a: setattr(a, "activation", -1), "MSS_ERR_BAD_STRUCT"),
    "width5": (lambda a: setattr(a, "width", 5), "MSS_ERR_BAD_SHAPE"),
    "batch0": (lambda a: setattr(a, "batch", 0), "MSS_ERR_BAD_SHAPE"),
    "state_null": (lambda a: setattr(a, "state", None), "MSS_ERR_NULL_POINTER"),
    "x_null": (lambda a: setattr(a, "x", None), "MSS_ERR_NULL_POINTER"),
    "neg_stride": (lambda a: a.out_stride.__setitem__(0, -1), "MSS_ERR_BAD_STRIDE"),
    "out_overlap": (lambda a: a.out_stride.__setitem__(1, 0), "MSS_ERR_BAD_STRIDE"),
    "misaligned_state": (lambda a: setattr(a, "state", fake(0) + 1), "MSS_ERR_MISALIGNED"),
    "out_is_state": (lambda a: setattr(a, "out", fake(0) + 8), "MSS_ERR_ALIASING"),
    "state_on_x": (lambda a: setattr(a, "state", fake(1)), "MSS_ERR_ALIASING"),
}


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(CONV_STEP_CASES))
def test_conv_step_argument_checks(case):
    fn, expect = CONV_STEP_CASES[case]
    a = conv_step_args()
    fn(a)
    assert _lib.lib().mss_causal_conv1d_update(ctypes.byref(a), None) == code(expect)


def bwd_args(ws=True):
    a = _lib.new_scan_bwd_args()
    a.io_dtype = _lib.MSS_F32
    a.batch, a.dim, a.seqlen, a.dstate = 2, 96, 100, 16
    x = (96 * 100, 100, 1)
    bc = (16 * 100, 100, 1)
    a.u, a.u_stride = fake(0), (ctypes.c_int64 * 3)(*x)
    a.delta_raw, a.delta_stride = fake(1), (ctypes.c_int64 * 3)(*x)
    a.A_log, a.A_log_stride = fake(2), (ctypes.c_int64 * 2)(16, 1)
    a.B, a.B_stride = fake(3), (ctypes.c_int64 * 3)(*bc)
    a.C, a.C_stride = fake(4), (ctypes.c_int64 * 3)(*bc)
    a.D = fake(5)
    a.z, a.z_stride = fake(6), (ctypes.c_int64 * 3)(*x)
    a.dt_bias = fake(7)
    a.delta_softplus = 1
    a.dout, a.dout_stride = fake(8), (ctypes.c_int64 * 3)(*x)
    a.du, a.du_stride = fake(9), (ctypes.c_int64 * 3)(*x)
    a.ddelta_raw, a.ddelta_stride = fake(10), (ctypes.c_int64 * 3)(*x)
    a.dA_log = fake(11)
    a.dB, a.dB_stride = fake(12), (ctypes.c_int64 * 3)(*bc)
    a.dC, a.dC_stride = fake(13), (ctypes.c_int64 * 3)(*bc)
    a.dD = fake(14)
    a.dz, a.dz_stride = fake(15), (ctypes.c_int64 * 3)(*x)
    a.ddt_bias = fake(16)
    if ws:
        st = ctypes.c_int(0)
        a.workspace = fake(17)
        a.workspace_bytes = _lib.lib().mss_selective_scan_bwd_workspace_size(ctypes.byref(a),
                                                                             ctypes.byref(st))
    return a


def test_bwd_workspace_size():
    lib = _lib.lib()
    a = bwd_args(ws=False)
    st = ctypes.c_int(-1)
    n = lib.mss_selective_scan_bwd_workspace_size(ctypes.byref(a), ctypes.byref(st))
    assert st.value == 0
    # the reverse walk takes 32-channel tiles: checkpoints 7 chunks x 2*3*32 padded
    # channels x 16 states; partials 2 rows x 4 chunk pairs (32 steps each, the
    # 100 steps rounded up) x 3 tiles x 32; per-row sums 2 x 96 x 18 (each
    # rounded up to 256 B)
    r = lambda v: (v + 255) // 256 * 256
    assert n == r(7 * 2 * 96 * 16 * 4) + r(2 * 4 * 3 * 32 * 32 * 4) + r(2 * 96 * 18 * 4)
    a.dstate = 0
    assert lib.mss_selective_scan_bwd_workspace_size(ctypes.byref(a), ctypes.byref(st)) == 0
    assert st.value == code("MSS_ERR_UNSUPPORTED_DSTATE")


BWD_CASES = {
    "struct_size": (lambda a: setattr(a, "struct_size", 4), "MSS_ERR_BAD_STRUCT"),
    "reverse_neg": (lambda a: setattr(a, "reverse", -1), "MSS_ERR_BAD_STRUCT"),
    "dtype": (lambda a: setattr(a, "io_dtype", 3), "MSS_ERR_UNSUPPORTED_DTYPE"),
    "seqlen0": (lambda a: setattr(a, "seqlen", 0), "MSS_ERR_BAD_SHAPE"),
    "dstate17": (lambda a: setattr(a, "dstate", 17), "MSS_ERR_UNSUPPORTED_DSTATE"),
    "dout_null": (lambda a: setattr(a, "dout", None), "MSS_ERR_NULL_POINTER"),
    "dB_null": (lambda a: setattr(a, "dB", None), "MSS_ERR_NULL_POINTER"),
    "dA_log_null": (lambda a: setattr(a, "dA_log", None), "MSS_ERR_NULL_POINTER"),
    "dz_without_z": (lambda a: setattr(a, "z", None), "MSS_ERR_NULL_POINTER"),
    "neg_stride": (lambda a: a.dout_stride.__setitem__(2, -1), "MSS_ERR_BAD_STRIDE"),
    "du_overlap": (lambda a: a.du_stride.__setitem__(1, 0), "MSS_ERR_BAD_STRIDE"),
    "dC_overlap": (lambda a: a.dC_stride.__setitem__(1, 0), "MSS_ERR_BAD_STRIDE"),
    "misaligned_dz": (lambda a: setattr(a, "dz", fake(15) + 2), "MSS_ERR_MISALIGNED"),
    "misaligned_dD": (lambda a: setattr(a, "dD", fake(14) + 1), "MSS_ERR_MISALIGNED"),
    "du_is_u": (lambda a: setattr(a, "du", fake(0)), "MSS_ERR_ALIASING"),
    "dB_is_B": (lambda a: setattr(a, "dB", fake(3)), "MSS_ERR_ALIASING"),
    "dz_on_dout": (lambda a: setattr(a, "dz", fake(8) + 400), "MSS_ERR_ALIASING"),
    "dD_in_dA_log": (lambda a: setattr(a, "dD", fake(11) + 8), "MSS_ERR_ALIASING"),
    "no_workspace": (lambda a: setattr(a, "workspace", None), "MSS_ERR_WORKSPACE_TOO_SMALL"),
    "short_workspace": (lambda a: setattr(a, "workspace_bytes", a.workspace_bytes - 1),
                        "MSS_ERR_WORKSPACE_TOO_SMALL"),
    "misaligned_workspace": (lambda a: setattr(a, "workspace", fake(17) + 64), "MSS_ERR_MISALIGNED"),
    "workspace_on_du": (lambda a: setattr(a, "workspace", fake(9)), "MSS_ERR_ALIASING"),
    "misaligned_chunk_states": (lambda a: setattr(a, "chunk_states", fake(18) + 4),
                                "MSS_ERR_MISALIGNED"),
    "chunk_states_on_du": (lambda a: setattr(a, "chunk_states", fake(9) + 512), "MSS_ERR_ALIASING"),
    "chunk_states_in_workspace": (lambda a: setattr(a, "chunk_states", fake(17) + 1024),
                                  "MSS_ERR_ALIASING"),
}


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(BWD_CASES))
def test_bwd_argument_checks(case):
    fn, expect = BWD_CASES[case]
    a = bwd_args()
    fn(a)
    assert _lib.lib().mss_selective_scan_bwd(ctypes.byref(a), None) == code(expect)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib(str(tmp_path / "missing.so"))


def cplx_args():
    a = _lib.new_scan_complex_args()
    a.batch, a.dim, a.seqlen, a.dstate = 2, 40, 50, 16
    x = (40 * 50, 50, 1)
    bc = (16 * 50, 50, 1)
    a.u, a.u_stride = fake(0), (ctypes.c_int64 * 3)(*x)
    a.delta_raw, a.delta_stride = fake(1), (ctypes.c_int64 * 3)(*x)
    a.A_log, a.A_log_stride = fake(2), (ctypes.c_int64 * 2)(16, 1)
    a.A_imag, a.A_imag_stride = fake(3), (ctypes.c_int64 * 2)(16, 1)
    a.B, a.B_stride = fake(4), (ctypes.c_int64 * 3)(*bc)
    a.C, a.C_stride = fake(5), (ctypes.c_int64 * 3)(*bc)
    a.D = fake(6)
    a.z, a.z_stride = fake(7), (ctypes.c_int64 * 3)(*x)
    a.dt_bias = fake(8)
    a.initial_state = fake(9)
    a.out, a.out_stride = fake(10), (ctypes.c_int64 * 3)(*x)
    a.final_state = fake(11)
    a.delta_softplus = 1
    return a


CPLX_CASES = {
    "null_struct": (None, "MSS_ERR_BAD_STRUCT"),
    "struct_size": (lambda a: setattr(a, "struct_size", 16), "MSS_ERR_BAD_STRUCT"),
    "reserved0": (lambda a: setattr(a, "reserved0", 1), "MSS_ERR_BAD_STRUCT"),
    "reserved1": (lambda a: setattr(a, "reserved1", 1), "MSS_ERR_BAD_STRUCT"),
    "seqlen0": (lambda a: setattr(a, "seqlen", 0), "MSS_ERR_BAD_SHAPE"),
    "dstate17": (lambda a: setattr(a, "dstate", 17), "MSS_ERR_UNSUPPORTED_DSTATE"),
    "A_imag_null": (lambda a: setattr(a, "A_imag", None), "MSS_ERR_NULL_POINTER"),
    "C_null": (lambda a: setattr(a, "C", None), "MSS_ERR_NULL_POINTER"),
    "neg_stride": (lambda a: a.B_stride.__setitem__(2, -1), "MSS_ERR_BAD_STRIDE"),
    "out_overlap": (lambda a: a.out_stride.__setitem__(1, 0), "MSS_ERR_BAD_STRIDE"),
    "misaligned_B": (lambda a: setattr(a, "B", fake(4) + 4), "MSS_ERR_MISALIGNED"),
    "misaligned_final": (lambda a: setattr(a, "final_state", fake(11) + 4), "MSS_ERR_MISALIGNED"),
    "out_is_u": (lambda a: setattr(a, "out", fake(0)), "MSS_ERR_ALIASING"),
    "final_on_C": (lambda a: setattr(a, "final_state", fake(5) + 64), "MSS_ERR_ALIASING"),
    "final_on_out": (lambda a: setattr(a, "final_state", fake(10) + 64), "MSS_ERR_ALIASING"),
    # this shape (6 tiles of 16 channels) is cut into time segments: it needs
    # a workspace, 256-byte aligned and clear of every tensor
    "no_workspace": (lambda a: None, "MSS_ERR_WORKSPACE_TOO_SMALL"),
    "workspace_short": (lambda a: (setattr(a, "workspace", fake(12)),
                                   setattr(a, "workspace_bytes", _cplx_ws(a) - 1)),
                        "MSS_ERR_WORKSPACE_TOO_SMALL"),
    "workspace_misaligned": (lambda a: (setattr(a, "workspace", fake(12) + 64),
                                        setattr(a, "workspace_bytes", _cplx_ws(a))),
                             "MSS_ERR_MISALIGNED"),
    "workspace_on_u": (lambda a: (setattr(a, "workspace", fake(0)),
                                  setattr(a, "workspace_bytes", _cplx_ws(a))), "MSS_ERR_ALIASING"),
}


def _cplx_ws(a):
    st = ctypes.c_int(-1)
    n = _lib.lib().mss_selective_scan_fwd_complex_workspace_size(ctypes.byref(a), ctypes.byref(st))
    assert st.value == 0
    return n


def test_complex_workspace_size_depends_on_shape_only():
    a = _lib.new_scan_complex_args()
    a.batch, a.dim, a.seqlen, a.dstate = 8, 5120, 4096, 16
    assert _cplx_ws(a) == 0                 # 2560 tiles: no time segments
    a.batch, a.dim, a.seqlen = 1, 256, 220500
    n = _cplx_ws(a)                          # 16 tiles: 80 segments of complex carries
    assert n >= 79 * 256 * 16 * 16 + 80 * 256 * 16 * 8
    a.dstate = 0
    st = ctypes.c_int(-1)
    assert _lib.lib().mss_selective_scan_fwd_complex_workspace_size(ctypes.byref(a),
                                                                    ctypes.byref(st)) == 0
    assert st.value == _lib.STATUS_CODE["MSS_ERR_UNSUPPORTED_DSTATE"]


@pytest.mark.skipif(HAS_GPU_NODE, reason="fake-pointer checks run only where no GPU is present")
@pytest.mark.parametrize("case", sorted(CPLX_CASES))
def test_complex_argument_checks(case):
    fn, expect = CPLX_CASES[case]
    a = None if fn is None else cplx_args()
    if fn is not None:
        fn(a)
    arg = ctypes.byref(a) if a is not None else None
    assert _lib.lib().mss_selective_scan_fwd_complex(arg, None) == code(expect)
