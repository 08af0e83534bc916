"""ctypes binding of libqmm.so (the C ABI in include/qmm.h).

Argument marshalling only: every computation runs in the HIP kernels.  If
the library has not been built this module raises instead of falling back
to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

# QMM_LIBRARY names another build of the same library (the host-sanitizer
# build of the CPU tests); by default the in-tree libqmm.so.
LIB_PATH = os.environ.get("QMM_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libqmm.so")

QMM_OK = 0
QMM_ERR_INVALID_ARG = 1
QMM_ERR_UNSUPPORTED = 2
QMM_ERR_WORKSPACE = 3
QMM_ERR_HIP = 4
QMM_WEIGHTS_TILED = 0x100  # bits flag: weights from qmm_repack_tiled
QMM_SCALES_TILED = 0x200  # bits flag: scales from qmm_repack_scales_tiled (biases unused)
QMM_GROUPED_SCRATCH_BYTES = 1 << 20  # static scratch of qmm_qgemm_grouped_noalloc

STATUS_NAMES = {0: "QMM_OK", 1: "QMM_ERR_INVALID_ARG", 2: "QMM_ERR_UNSUPPORTED",
                3: "QMM_ERR_WORKSPACE", 4: "QMM_ERR_HIP"}


class QmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class GemvProblem(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("x", C.c_void_p), ("y", C.c_void_p), ("n", C.c_int32), ("k", C.c_int32)]


class GemmProblem(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p),
                ("x", C.c_void_p), ("y", C.c_void_p), ("m", C.c_int32), ("n", C.c_int32),
                ("k", C.c_int32)]


P, I, SZ = C.c_void_p, C.c_int, C.c_size_t

SIGNATURES = {
    "qmm_version": (I, []),
    "qmm_last_error": (C.c_char_p, []),
    "qmm_qgemv": (I, [P, P, P, P, P, I, I, I, I, P]),
    "qmm_qgemv_batched_plan": (I, [C.POINTER(GemvProblem), I, I, I, P, SZ, C.POINTER(SZ)]),
    "qmm_qgemv_batched": (I, [P, P, P]),
    "qmm_qgemm_workspace_size": (SZ, [I, I, I, I, I]),
    "qmm_qgemm": (I, [P, P, P, P, P, I, I, I, I, I, P, SZ, P]),
    "qmm_qgemm_batched_plan": (I, [C.POINTER(GemmProblem), I, I, I, P, SZ, C.POINTER(SZ),
                                   C.POINTER(SZ)]),
    "qmm_qgemm_batched": (I, [P, P, P, SZ, P]),
    "qmm_qgemm_grouped_workspace_size": (SZ, [I, I, I, I, I, I, I]),
    "qmm_qgemm_grouped": (I, [P, P, P, P, I, P, P, I, I, I, I, I, I, I, P, SZ, P]),
    "qmm_qgemm_grouped_noalloc": (I, [P, P, P, P, I, P, P, I, I, I, I, I, I, I, P]),
    "qmm_moe_route_size": (SZ, [I, I, I]),
    "qmm_moe_route": (I, [P, I, I, I, P, SZ, P]),
    "qmm_qgemm_grouped_routed": (I, [P, P, P, P, I, P, SZ, P, I, I, I, I, I, I, I, P]),
    "qmm_moe_gate_up_swiglu": (I, [P, P, P, P, P, P, P, P, SZ, P, I, I, I, I, I, I, I, P]),
    "qmm_moe_combine": (I, [P, P, P, I, I, I, P]),
    "qmm_convert_bf16": (I, [P, P, SZ, P]),
    "qmm_repack_tiled": (I, [P, P, I, I, I, P]),
    "qmm_repack_scales_tiled": (I, [P, P, P, I, I, P]),
    "qmm_quantize": (I, [P, P, P, P, I, I, I, I, P]),
    "qmm_unpack_codes": (I, [P, P, I, I, I, P]),
    "qmm_dequant": (I, [P, P, P, P, I, I, I, I, I, P]),
}

_lib = None


def lib() -> C.CDLL:
    """Load libqmm.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m quantized_matmul_qgemv_amd.build`")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().qmm_last_error().decode()


def check(status: int) -> None:
    if status != QMM_OK:
        raise QmmError(status, last_error())
