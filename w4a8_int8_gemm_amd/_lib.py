"""ctypes loader for libw4a8.so, the HIP library (argument marshalling only).

The library is built in-tree by ``w4a8_int8_gemm_amd/build.py``; if no built
library is present it is built on first use.  There is no fallback: when the
library cannot be built or loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import enum
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a8.so")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

# name -> argument types (all return int32 status unless listed in _RESTYPES)
_SIGNATURES = {
    "w4a8_is_available": [],
    "w4a8_status_string": [ctypes.c_int],
    "w4a8_last_error": [],
    "quantize_act": [_vp, _i64, _i64, _i32, _vp, _vp, _vp],
    "quantize_weight_int8": [_vp, _i64, _i64, _i32, _vp, _vp, _vp],
    "pack_weight_int4": [_vp, _i64, _i64, _i32, _vp, _vp, _vp],
    "w8a8_gemm_pc": [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "w8a8_gemm_pg": [_vp, _vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp],
    "w4a8_gemm": [_vp, _vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp],
    "int8_mv": [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp],
    "w8a8_mv_pg": [_vp, _vp, _vp, _i32, _vp, _i64, _i64, _vp],
    "w4a8_mv": [_vp, _vp, _vp, _i32, _vp, _i64, _i64, _vp],
    "linear_workspace_size": [ctypes.c_int, _i64, _i64, _i32],
    "linear": [ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _vp, _sz, _vp],
    "linear_noalloc": [ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _vp],
    "w8a8_gemm_i32": [_vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "w8a8_gemm_pg_partials": [_vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp],
    "w4a8_gemm_partials": [_vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp],
    "w8a16_gemm": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp],
    "w4a16_gemm": [_vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp],
    "gemm_tile_config": [ctypes.c_int, _i64, _i64, _i64, _i32, ctypes.POINTER(_i64)],
}
_RESTYPES = {
    "w4a8_is_available": ctypes.c_int,
    "w4a8_status_string": ctypes.c_char_p,
    "w4a8_last_error": ctypes.c_char_p,
    "linear_workspace_size": _sz,
}


class Status(enum.IntEnum):
    OK = 0
    ERR_INVALID_ARG = 1
    ERR_SHAPE = 2
    ERR_ALIGNMENT = 3
    ERR_DEVICE = 4
    ERR_LAUNCH = 5
    ERR_WORKSPACE = 6


class Mode(enum.IntEnum):
    W8A8_PC = 0
    W8A8_PG = 1
    W4A8 = 2


class GemmOp(enum.IntEnum):
    GEMM_PC = 0
    GEMM_PG = 1
    GEMM_W4A8 = 2
    GEMM_I32 = 3
    PG_PARTIALS = 4
    W4A8_PARTIALS = 5


class W4A8Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = Status(status)
        super().__init__(f"{self.status.name}: {detail}")


_lib = None


def lib():
    """The loaded library (built first if nothing is built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, ctypes.c_int)
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise W4A8Error(status, lib().w4a8_last_error().decode())
