"""ctypes loader for libusw.so (argument marshalling only).

The shared library is built in-tree by ``unstructured_sparse_weight_amd.build``.
Loading fails loudly when it is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# USW_LIB_PATH names another build of the same library (the sanitizer
# build of the host code that the test suite runs the C-ABI tests against).
LIB_PATH = os.environ.get("USW_LIB_PATH") or os.path.join(_PKG, "libusw.so")

USW_OK = 0
USW_VAL_F16 = 1
USW_VAL_I4 = 2
USW_VAL_I2 = 3
USW_OUT_F16 = 1
USW_OUT_F32 = 3

STATUS_NAMES = {
    0: "OK", -1: "NULL_ARG", -2: "BAD_SHAPE", -3: "BAD_DTYPE", -4: "BAD_N", -5: "UNSUPPORTED",
    -6: "MISALIGNED", -7: "WORKSPACE", -8: "CORRUPT", -9: "HIP", -10: "CAPACITY",
}

# Every symbol include/usw.h declares.
EXPORTED = (
    "usw_abi_version", "usw_status_str", "usw_encode_query", "usw_encode", "usw_validate",
    "usw_encode_device_index", "usw_encode_device_values",
    "usw_spmm_workspace", "usw_spmm", "usw_spmm_workspace_ex", "usw_spmm_ex", "usw_spmm_counter_bytes",
    "usw_spmm_noalloc", "usw_probe_read",
    "usw_union_encode_query", "usw_union_encode", "usw_union_validate", "usw_union_reorder",
    "usw_union_encode_reordered_query", "usw_union_encode_reordered",
    "usw_union_encode_device_index", "usw_union_encode_device_values", "usw_union_spmm_workspace",
    "usw_union_spmm_counter_bytes", "usw_union_spmm",
    "usw_cbc_encode_query", "usw_cbc_encode", "usw_cbc_validate",
    "usw_cbc_encode_device_index", "usw_cbc_encode_device_values", "usw_cbc_spmspv_workspace", "usw_cbc_spmspv",
)


class UswError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


class UswFmt(ctypes.Structure):
    """Mirror of ``usw_fmt``."""
    _fields_ = [
        ("M", ctypes.c_int32), ("K", ctypes.c_int32),
        ("gt_m", ctypes.c_int32), ("gt_k", ctypes.c_int32),
        ("val_type", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("nnz", ctypes.c_int64),
        ("bitmaps", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
        ("values", ctypes.c_void_p), ("scales", ctypes.c_void_p),
    ]


class UswUnionFmt(ctypes.Structure):
    """Mirror of ``usw_union_fmt``."""
    _fields_ = [
        ("M", ctypes.c_int32), ("K", ctypes.c_int32),
        ("lt_m", ctypes.c_int32), ("lt_k", ctypes.c_int32),
        ("r_a", ctypes.c_int32), ("c_a", ctypes.c_int32),
        ("val_type", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("payload", ctypes.c_int64),
        ("bitmaps", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
        ("values", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("rowmap", ctypes.c_void_p),
    ]


class UswCbcFmt(ctypes.Structure):
    """Mirror of ``usw_cbc_fmt``."""
    _fields_ = [
        ("M", ctypes.c_int32), ("K", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("val_type", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("nnz_padded", ctypes.c_int64),
        ("bitmaps", ctypes.c_void_p), ("tile_offsets", ctypes.c_void_p),
        ("colinfo", ctypes.c_void_p), ("values", ctypes.c_void_p),
    ]


_lib = None


def _declare(lib):
    c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    P = ctypes.POINTER
    lib.usw_abi_version.restype = c_i32
    lib.usw_abi_version.argtypes = []
    lib.usw_status_str.restype = ctypes.c_char_p
    lib.usw_status_str.argtypes = [c_i32]
    lib.usw_encode_query.restype = c_i32
    lib.usw_encode_query.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, P(c_i64),
                                     P(c_sz), P(c_sz), P(c_sz), P(c_sz), P(c_sz)]
    lib.usw_encode.restype = c_i32
    lib.usw_encode.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]
    lib.usw_validate.restype = c_i32
    lib.usw_validate.argtypes = [P(UswFmt)]
    lib.usw_spmm_workspace.restype = c_i32
    lib.usw_spmm_workspace.argtypes = [P(UswFmt), c_i32, P(c_sz)]
    lib.usw_spmm.restype = c_i32
    lib.usw_spmm.argtypes = [P(UswFmt), c_vp, c_vp, c_i32, c_i32, c_vp, c_sz, c_vp]
    lib.usw_spmm_workspace_ex.restype = c_i32
    lib.usw_spmm_workspace_ex.argtypes = [P(UswFmt), c_i32, c_i32, P(c_sz)]
    lib.usw_spmm_ex.restype = c_i32
    lib.usw_spmm_ex.argtypes = [P(UswFmt), c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]
    lib.usw_spmm_noalloc.restype = c_i32
    lib.usw_spmm_noalloc.argtypes = [P(UswFmt), c_vp, c_vp, c_i32, c_i32, c_i32, c_vp]
    lib.usw_spmm_counter_bytes.restype = c_i32
    lib.usw_spmm_counter_bytes.argtypes = [P(UswFmt), c_i32, c_i32, P(c_sz)]
    lib.usw_probe_read.restype = c_i32
    lib.usw_probe_read.argtypes = [ctypes.c_void_p, c_sz, ctypes.c_void_p, ctypes.c_void_p]
    lib.usw_union_encode_query.restype = c_i32
    lib.usw_union_encode_query.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, P(c_i64),
                                           P(c_sz), P(c_sz), P(c_sz), P(c_sz), P(c_sz)]
    lib.usw_union_encode.restype = c_i32
    lib.usw_union_encode.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                     c_sz, c_vp]
    lib.usw_union_validate.restype = c_i32
    lib.usw_union_validate.argtypes = [P(UswUnionFmt)]
    lib.usw_union_encode_reordered_query.restype = c_i32
    lib.usw_union_encode_reordered_query.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                     c_vp, P(c_i64), P(c_sz), P(c_sz)]
    lib.usw_union_encode_reordered.restype = c_i32
    lib.usw_union_encode_reordered.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                               c_vp, c_vp, c_vp, c_sz, c_vp, c_vp]
    lib.usw_union_spmm_workspace.restype = c_i32
    lib.usw_union_spmm_workspace.argtypes = [P(UswUnionFmt), c_i32, c_i32, P(c_sz)]
    lib.usw_union_spmm_counter_bytes.restype = c_i32
    lib.usw_union_spmm_counter_bytes.argtypes = [P(UswUnionFmt), c_i32, c_i32, P(c_sz)]
    lib.usw_union_spmm.restype = c_i32
    lib.usw_union_spmm.argtypes = [P(UswUnionFmt), c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]
    lib.usw_cbc_encode_query.restype = c_i32
    lib.usw_cbc_encode_query.argtypes = [c_vp, c_vp, c_i32, c_i32, P(c_i64), P(c_i64), P(c_sz), P(c_sz), P(c_sz),
                                         P(c_sz)]
    lib.usw_cbc_encode.restype = c_i32
    lib.usw_cbc_encode.argtypes = [c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz]
    lib.usw_cbc_validate.restype = c_i32
    lib.usw_cbc_validate.argtypes = [P(UswCbcFmt)]
    lib.usw_cbc_spmspv_workspace.restype = c_i32
    lib.usw_cbc_spmspv_workspace.argtypes = [P(UswCbcFmt), c_i32, P(c_sz), P(c_sz)]
    lib.usw_cbc_spmspv.restype = c_i32
    lib.usw_cbc_spmspv.argtypes = [P(UswCbcFmt), c_vp, c_vp, c_i32, ctypes.c_float, c_i32, c_vp, c_sz, c_vp]
    lib.usw_union_encode_device_index.restype = c_i32
    lib.usw_union_encode_device_index.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                                  c_vp, c_vp, c_vp]
    lib.usw_union_encode_device_values.restype = c_i32
    lib.usw_union_encode_device_values.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp,
                                                   c_vp, c_vp, c_i64, c_vp, c_sz, c_vp]
    lib.usw_cbc_encode_device_index.restype = c_i32
    lib.usw_cbc_encode_device_index.argtypes = [c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
    lib.usw_cbc_encode_device_values.restype = c_i32
    lib.usw_cbc_encode_device_values.argtypes = [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_sz, c_vp]
    lib.usw_union_reorder.restype = c_i32
    lib.usw_union_reorder.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]
    lib.usw_encode_device_index.restype = c_i32
    lib.usw_encode_device_index.argtypes = [c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
    lib.usw_encode_device_values.restype = c_i32
    lib.usw_encode_device_values.argtypes = [c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp,
                                             c_sz, c_vp]
    return lib


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m unstructured_sparse_weight_amd.build` "
                "(there is no fallback implementation)")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def check(status: int, where: str) -> None:
    if status != USW_OK:
        raise UswError(status, where, lib().usw_status_str(status).decode())
