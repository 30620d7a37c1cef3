"""ctypes loader for ``libkda.so`` (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

# Every symbol include/kda.h declares.
EXPORTS = ("kda_fwd", "kda_fwd_ex", "kda_fwd_scan", "kda_fwd_scan_static",
           "kda_fwd_scan_workspace_bytes", "kda_status_string", "kda_fwd_kernel",
           "kda_abi_version")
SCAN_STATIC_BYTES = 32 << 20  # KDA_SCAN_STATIC_BYTES
ABI_VERSION = 4

# kda_status codes (include/kda.h)
KDA_OK = 0
KDA_ERR_NULL_POINTER = 1
KDA_ERR_HEAD_DIM = 2
KDA_ERR_LOWER_BOUND = 3
KDA_ERR_VARLEN_BATCH = 4
KDA_ERR_STATE_DTYPE = 5
KDA_ERR_ALIAS = 6
KDA_ERR_SIZE = 7
KDA_ERR_SCALE = 8
KDA_ERR_LAUNCH = 9
KDA_ERR_WORKSPACE = 10
KDA_ERR_ALIGNMENT = 11
KDA_ERR_OPTION = 12

# kda_dtype codes
KDA_DTYPE_NONE = 0
KDA_DTYPE_BF16 = 1
KDA_DTYPE_FP32 = 2

# kda_options fields
KDA_KERNEL_AUTO, KDA_KERNEL_CHUNKED, KDA_KERNEL_RECURRENT, KDA_KERNEL_SINGLE = 0, 1, 2, 3
KDA_INVERSE_SUBSTITUTION, KDA_INVERSE_NEUMANN = 0, 1
KDA_SIGMOID_EXP2, KDA_SIGMOID_TANH = 0, 1


class Options(ctypes.Structure):
    """struct kda_options"""
    _fields_ = [("kernel", ctypes.c_int32), ("inverse", ctypes.c_int32),
                ("sigmoid", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KdaLibraryMissing(RuntimeError):
    """libkda.so has not been built (there is no other implementation)."""


_lib = None


def load() -> ctypes.CDLL:
    """Load libkda.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise KdaLibraryMissing(
            f"{LIBRARY} is missing; build it with `python -m gated_delta_rule_36_amd.build`")
    lib = ctypes.CDLL(LIBRARY)
    p, i64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
    lib.kda_fwd.argtypes = [p, p, p, p, p, d, p, p, p, d, p, ctypes.c_int, p, ctypes.c_int,
                            p, i64, i64, i64, i64, i64, i64, p]
    lib.kda_fwd.restype = ctypes.c_int
    opt = ctypes.POINTER(Options)
    lib.kda_fwd_ex.argtypes = [p, p, p, p, p, d, p, p, p, d, p, ctypes.c_int, p, ctypes.c_int,
                               p, i64, i64, i64, i64, i64, i64, opt, p]
    lib.kda_fwd_ex.restype = ctypes.c_int
    lib.kda_fwd_scan.argtypes = [p, p, p, p, p, d, p, p, p, d, p, ctypes.c_int, p, ctypes.c_int,
                                 p, i64, i64, i64, i64, i64, i64, i64, p, i64, opt, p]
    lib.kda_fwd_scan.restype = ctypes.c_int
    lib.kda_fwd_scan_static.argtypes = [p, p, p, p, p, d, p, p, p, d, p, ctypes.c_int, p,
                                        ctypes.c_int, p, i64, i64, i64, i64, i64, i64, i64, opt, p]
    lib.kda_fwd_scan_static.restype = ctypes.c_int
    lib.kda_fwd_scan_workspace_bytes.argtypes = [p, i64, i64, i64, i64, i64]
    lib.kda_fwd_scan_workspace_bytes.restype = i64
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_fwd_kernel.argtypes = [i64, ctypes.c_int, opt]
    lib.kda_fwd_kernel.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    if lib.kda_abi_version() != ABI_VERSION:
        raise KdaLibraryMissing(f"{LIBRARY} has ABI {lib.kda_abi_version()}, expected {ABI_VERSION}")
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().kda_status_string(code).decode()
