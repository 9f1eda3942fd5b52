"""ctypes loader of libqlin.so and the C signatures of include/qlin.h.

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlin.so")

p = C.c_void_p
i32 = C.c_int32
i64 = C.c_int64
f32 = C.c_float

# name -> (restype, argtypes); mirrors include/qlin.h
SIGNATURES = {
    "qlin_abi_version": (i32, []),
    "qlin_status_string": (C.c_char_p, [i32]),
    "qlin_last_error": (C.c_char_p, []),
    "qlin_outlier_ld": (i32, [i32]),
    "qlin_quant_act": (i32, [p, i64, i64, p, p, p, p, i32, p, p, p, p]),
    "qlin_hadamard_offset": (i32, [p, i64, i64, p, i32, p, p, p, p, p, p]),
    "qlin_hadamard_offset_group": (i32, [p, i64, i64, p, i32, p, p, p, p, p, p]),
    "qlin_momentum_update": (i32, [p, i64, i64, p, i32, p, f32, p, p, p, p]),
    "qlin_momentum_work_bytes": (C.c_size_t, [i64, i32]),
    "qlin_momentum_update_noalloc": (i32, [p, i64, i64, p, i32, p, f32, p, p, p]),
    "qlin_quaff_momentum_quant": (i32, [p, i64, i64, p, i32, p, f32, p, p, p, p, p, p, p]),
    "qlin_quaff_momentum_quant_work_bytes": (C.c_size_t, [i64, i32]),
    "qlin_quant_weight_sym": (i32, [p, i64, i64, i32, p, p, p]),
    "qlin_quant_weight_group": (i32, [p, i64, i64, i32, p, p, p, p, p]),
    "qlin_quant_weight_offq": (i32, [p, i64, i64, p, i32, p, p, p, p, p]),
    "qlin_weight_row_absmax": (i32, [p, i64, i64, p, p]),
    "qlin_weight_colsum_group": (i32, [p, i64, i64, i32, p, p]),
    "qlin_packed_bytes": (C.c_size_t, [i32, i64, i64]),
    "qlin_pack_weight": (i32, [i32, p, i64, i64, p, p]),
    "qlin_gemm_w8a8": (i32, [p, p, p, p, i64, i64, i64, p, i32, p, p, p, p]),
    "qlin_gemm_w4a8": (i32, [p, p, p, p, p, i32, i64, i64, i64, p, p, p, p]),
    "qlin_gemm_w4a8_work_bytes": (C.c_size_t, [i64, i64, i64, i32]),
    "qlin_gemm_w4a4": (i32, [p, p, p, p, p, p, p, p, i64, i64, i64, p, p, p]),
    "qlin_gemm_w4a4_group": (i32, [p, p, p, p, p, p, p, p, i64, i64, i64, p, p, p]),
    "qlin_outlier_comp": (i32, [p, p, i32, p, i64, i64, p, p]),
    "qlin_pca_select": (i32, [p, i64, i64, i64, p, p, p]),
    "qlin_pca_leading_eigvec": (i32, [p, i64, i64, i32, C.c_double, p, p, p, p, p]),
    "qlin_pca_fold_weight": (i32, [p, i64, i64, p, p, p, p]),
    "qlin_pca_rotate": (i32, [p, i64, i64, p, p, p]),
    "qlin_quaff_backward": (i32, [p, i64, i64, i64, p, p, p, p, p, i32, p, p, p, p, p, p, p]),
}

QLIN_OK = 0
QLIN_ERR_INVALID_ARG = 1
QLIN_ERR_SHAPE = 2
QLIN_ERR_ALIGN = 3
QLIN_ERR_UNSUPPORTED = 4
QLIN_ERR_HIP = 5
QLIN_LAYOUT_W8 = 1
QLIN_LAYOUT_W4S = 2
QLIN_LAYOUT_W4U = 3
QLIN_LAYOUT_WO = 4
QLIN_LAYOUT_W8T = 5

_lib = None


def load() -> C.CDLL:
    """The loaded libqlin (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python outlier_aware_bit_amd/build.py` "
                "(hipcc --offload-arch=gfx950); there is no fallback implementation")
        # One HIP runtime per process: torch ships its own libamdhip64 (same
        # SONAME as ROCm's).  Loading torch first makes libqlin bind to the
        # runtime that owns torch's allocations and streams; loading libqlin
        # first would pull in a second runtime beside torch's.
        import torch  # noqa: F401
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class QlinError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        self.status = status
        super().__init__(f"{fn}: {lib.qlin_status_string(status).decode()}: {lib.qlin_last_error().decode()}")


def check(fn: str, status: int) -> None:
    if status != QLIN_OK:
        raise QlinError(fn, status)
