"""ctypes view of include/mss.h: structs, status codes and the loaded library.

Argument marshalling only.  Importing this module does not load libmss; the
first call of ``lib()`` does, and raises if the library has not been built.
There is no fallback path: without libmss.so the package cannot compute.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmss.so")

MSS_ABI_VERSION = 5
MSS_MAX_DSTATE = 16
MSS_STATE_CHUNK = 16
MSS_MAX_CONV_WIDTH = 4
MSS_NOALLOC_SCRATCH_BYTES = 16 << 20
MSS_F32 = 0
MSS_BF16 = 1
MSS_ACT_NONE = 0
MSS_ACT_SILU = 1

STATUS = {
    0: "MSS_OK",
    1: "MSS_ERR_NULL_POINTER",
    2: "MSS_ERR_BAD_SHAPE",
    3: "MSS_ERR_BAD_STRIDE",
    4: "MSS_ERR_UNSUPPORTED_DTYPE",
    5: "MSS_ERR_UNSUPPORTED_DSTATE",
    6: "MSS_ERR_MISALIGNED",
    7: "MSS_ERR_WORKSPACE_TOO_SMALL",
    8: "MSS_ERR_ALIASING",
    9: "MSS_ERR_BAD_STRUCT",
    10: "MSS_ERR_HIP",
    11: "MSS_ERR_SCRATCH_LIMIT",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

EXPORTS = ("mss_abi_version", "mss_status_string", "mss_selective_scan_workspace_size",
           "mss_selective_scan_fwd", "mss_selective_state_update", "mss_causal_conv1d_fwd",
           "mss_causal_conv1d_update", "mss_selective_scan_bwd_workspace_size",
           "mss_selective_scan_bwd", "mss_selective_scan_fwd_complex",
           "mss_selective_scan_fwd_noalloc", "mss_selective_scan_fwd_complex_workspace_size")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class ScanArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("io_dtype", _i32),
        ("batch", _i64), ("dim", _i64), ("seqlen", _i64), ("dstate", _i64),
        ("u", _vp), ("u_stride", _i64 * 3),
        ("delta_raw", _vp), ("delta_stride", _i64 * 3),
        ("A_log", _vp), ("A_log_stride", _i64 * 2),
        ("B", _vp), ("B_stride", _i64 * 3),
        ("C", _vp), ("C_stride", _i64 * 3),
        ("D", _vp),
        ("z", _vp), ("z_stride", _i64 * 3),
        ("dt_bias", _vp),
        ("initial_state", _vp),
        ("out", _vp), ("out_stride", _i64 * 3),
        ("final_state", _vp),
        ("chunk_states", _vp),
        ("delta_softplus", _i32), ("reverse", _i32),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


class StepArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("io_dtype", _i32),
        ("batch", _i64), ("dim", _i64), ("dstate", _i64),
        ("state", _vp),
        ("u", _vp), ("u_stride", _i64 * 2),
        ("delta_raw", _vp), ("delta_stride", _i64 * 2),
        ("A_log", _vp), ("A_log_stride", _i64 * 2),
        ("B", _vp), ("B_stride", _i64 * 2),
        ("C", _vp), ("C_stride", _i64 * 2),
        ("D", _vp),
        ("z", _vp), ("z_stride", _i64 * 2),
        ("dt_bias", _vp),
        ("out", _vp), ("out_stride", _i64 * 2),
        ("delta_softplus", _i32), ("reserved0", _i32),
    ]


class ScanBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("io_dtype", _i32),
        ("batch", _i64), ("dim", _i64), ("seqlen", _i64), ("dstate", _i64),
        ("u", _vp), ("u_stride", _i64 * 3),
        ("delta_raw", _vp), ("delta_stride", _i64 * 3),
        ("A_log", _vp), ("A_log_stride", _i64 * 2),
        ("B", _vp), ("B_stride", _i64 * 3),
        ("C", _vp), ("C_stride", _i64 * 3),
        ("D", _vp),
        ("z", _vp), ("z_stride", _i64 * 3),
        ("dt_bias", _vp),
        ("initial_state", _vp),
        ("delta_softplus", _i32), ("reverse", _i32),
        ("dout", _vp), ("dout_stride", _i64 * 3),
        ("dfinal_state", _vp),
        ("chunk_states", _vp),
        ("du", _vp), ("du_stride", _i64 * 3),
        ("ddelta_raw", _vp), ("ddelta_stride", _i64 * 3),
        ("dA_log", _vp),
        ("dB", _vp), ("dB_stride", _i64 * 3),
        ("dC", _vp), ("dC_stride", _i64 * 3),
        ("dD", _vp),
        ("dz", _vp), ("dz_stride", _i64 * 3),
        ("ddt_bias", _vp),
        ("dinitial_state", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


def new_scan_bwd_args() -> ScanBwdArgs:
    a = ScanBwdArgs()
    a.struct_size = ctypes.sizeof(ScanBwdArgs)
    return a


class ConvArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("io_dtype", _i32),
        ("batch", _i64), ("dim", _i64), ("seqlen", _i64), ("width", _i64),
        ("x", _vp), ("x_stride", _i64 * 3),
        ("weight", _vp), ("weight_stride", _i64 * 2),
        ("bias", _vp),
        ("initial_state", _vp),
        ("out", _vp), ("out_stride", _i64 * 3),
        ("final_state", _vp),
        ("activation", _i32), ("reserved0", _i32),
    ]


class ConvStepArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("io_dtype", _i32),
        ("batch", _i64), ("dim", _i64), ("width", _i64),
        ("state", _vp),
        ("x", _vp), ("x_stride", _i64 * 2),
        ("weight", _vp), ("weight_stride", _i64 * 2),
        ("bias", _vp),
        ("out", _vp), ("out_stride", _i64 * 2),
        ("activation", _i32), ("reserved0", _i32),
    ]


def new_conv_args() -> ConvArgs:
    a = ConvArgs()
    a.struct_size = ctypes.sizeof(ConvArgs)
    return a


def new_conv_step_args() -> ConvStepArgs:
    a = ConvStepArgs()
    a.struct_size = ctypes.sizeof(ConvStepArgs)
    return a


def new_scan_args() -> ScanArgs:
    a = ScanArgs()
    a.struct_size = ctypes.sizeof(ScanArgs)
    return a


class ScanComplexArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("reserved0", _i32),
        ("batch", _i64), ("dim", _i64), ("seqlen", _i64), ("dstate", _i64),
        ("u", _vp), ("u_stride", _i64 * 3),
        ("delta_raw", _vp), ("delta_stride", _i64 * 3),
        ("A_log", _vp), ("A_log_stride", _i64 * 2),
        ("A_imag", _vp), ("A_imag_stride", _i64 * 2),
        ("B", _vp), ("B_stride", _i64 * 3),
        ("C", _vp), ("C_stride", _i64 * 3),
        ("D", _vp),
        ("z", _vp), ("z_stride", _i64 * 3),
        ("dt_bias", _vp),
        ("initial_state", _vp),
        ("out", _vp), ("out_stride", _i64 * 3),
        ("final_state", _vp),
        ("delta_softplus", _i32), ("reserved1", _i32),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
    ]


def new_scan_complex_args() -> ScanComplexArgs:
    a = ScanComplexArgs()
    a.struct_size = ctypes.sizeof(ScanComplexArgs)
    return a


def new_step_args() -> StepArgs:
    a = StepArgs()
    a.struct_size = ctypes.sizeof(StepArgs)
    return a


class MssError(RuntimeError):
    """A libmss call returned a status other than MSS_OK."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.name = STATUS.get(code, str(code))


_LIB = None


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.mss_abi_version.argtypes = []
    lib.mss_abi_version.restype = ctypes.c_int
    lib.mss_status_string.argtypes = [ctypes.c_int]
    lib.mss_status_string.restype = ctypes.c_char_p
    lib.mss_selective_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs),
                                                      ctypes.POINTER(ctypes.c_int)]
    lib.mss_selective_scan_workspace_size.restype = ctypes.c_size_t
    lib.mss_selective_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _vp]
    lib.mss_selective_scan_fwd.restype = ctypes.c_int
    lib.mss_selective_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _vp]
    lib.mss_selective_scan_fwd_noalloc.restype = ctypes.c_int
    lib.mss_selective_state_update.argtypes = [ctypes.POINTER(StepArgs), _vp]
    lib.mss_selective_state_update.restype = ctypes.c_int
    lib.mss_selective_scan_fwd_complex.argtypes = [ctypes.POINTER(ScanComplexArgs), _vp]
    lib.mss_selective_scan_fwd_complex.restype = ctypes.c_int
    lib.mss_selective_scan_fwd_complex_workspace_size.argtypes = [
        ctypes.POINTER(ScanComplexArgs), ctypes.POINTER(ctypes.c_int)]
    lib.mss_selective_scan_fwd_complex_workspace_size.restype = ctypes.c_size_t
    lib.mss_selective_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(ScanBwdArgs),
                                                          ctypes.POINTER(ctypes.c_int)]
    lib.mss_selective_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mss_selective_scan_bwd.argtypes = [ctypes.POINTER(ScanBwdArgs), _vp]
    lib.mss_selective_scan_bwd.restype = ctypes.c_int
    lib.mss_causal_conv1d_fwd.argtypes = [ctypes.POINTER(ConvArgs), _vp]
    lib.mss_causal_conv1d_fwd.restype = ctypes.c_int
    lib.mss_causal_conv1d_update.argtypes = [ctypes.POINTER(ConvStepArgs), _vp]
    lib.mss_causal_conv1d_update.restype = ctypes.c_int
    return lib


def lib(path: str = LIB_PATH) -> ctypes.CDLL:
    """The loaded libmss (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"libmss.so is not built ({path}); run `python -c 'import __graft_entry__ as g; "
                "g.build()'` or `python -m mamba_selective_scan_amd.build` first")
        l = _bind(ctypes.CDLL(path))
        v = l.mss_abi_version()
        if v != MSS_ABI_VERSION:
            raise RuntimeError(f"libmss ABI version {v}, binding expects {MSS_ABI_VERSION}")
        _LIB = l
    return _LIB


def check(code: int) -> None:
    if code != 0:
        msg = lib().mss_status_string(code).decode()
        raise MssError(code, msg)
