"""CPU oracle for the W8A8 / W4A8 int8 linear layer -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The GPU library never calls
it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain loops, see its header for the
passages each function follows); this module marshals numpy arrays and
composes the steps in the order the pages give them:

  [P1] "Apple Silicon의 AI 한계치는 당신의 생각보다 높습니다", section
       "INT8 TensorOps 커널 설계": scale from a min/max reduction, INT8
       activation codes, INT8 GEMM with INT32 accumulation, rescale by the
       product of scales to FP16.
  [P2] "cider: Apple Silicon M5 INT8 TensorOps ... W8A8 SDK", section on
       quantization modes (per-token INT8 activations; symmetric INT8 or
       uint8-packed INT4 weights; per-channel, gs=128 and gs=64 groups) and
       section on path selection (M == 1 goes to the matrix-vector kernel,
       larger M to the GEMM).

fp16 values travel as ``numpy.float16`` arrays (their bits are what the C
side reads).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib():
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        L.oracle_w8a16.argtypes = [_u16p, _i8p, _f32p, _i64, _i64, _i64, _u16p, _f64p]
        L.oracle_w8a16.restype = None
        L.oracle_w4a16.argtypes = [_u16p, _i8p, _f32p, _i64, _i64, _i64, _i64, _u16p, _f64p]
        L.oracle_w4a16.restype = None
        L.oracle_quantize_sym.argtypes = [_u16p, _i64, _i64, _i64, ctypes.c_int32, _i8p, _f32p]
        L.oracle_quantize_sym.restype = ctypes.c_int
        L.oracle_pack_int4.argtypes = [_i8p, _i64, _i64, _u8p]
        L.oracle_pack_int4.restype = ctypes.c_int
        L.oracle_unpack_int4.argtypes = [_u8p, _i64, _i64, _i8p]
        L.oracle_unpack_int4.restype = ctypes.c_int
        L.oracle_gemm_i32.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i32p]
        L.oracle_gemm_i32.restype = ctypes.c_int
        L.oracle_gemm_partials.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i64, _i32p]
        L.oracle_gemm_partials.restype = ctypes.c_int
        L.oracle_epilogue_pc.argtypes = [_i32p, _f32p, _f32p, _i64, _i64, _u16p]
        L.oracle_epilogue_pc.restype = None
        L.oracle_epilogue_pg.argtypes = [_i32p, _f32p, _f32p, _i64, _i64, _i64, _u16p, _f64p]
        L.oracle_epilogue_pg.restype = None
        L.oracle_epilogue_w4a8.argtypes = [_i32p, _f32p, _f32p, _i64, _i64, _i64, _u16p, _f64p]
        L.oracle_epilogue_w4a8.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, typ):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(typ)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's parallel loops (timing: one core against all)."""
    lib().oracle_set_num_threads(int(n))


# ----------------------------------------------------------------------------- fp16 rounding

def f64_to_f16(values) -> np.ndarray:
    """Round fp64 values to fp16 (nearest, ties to even) one by one."""
    v = np.asarray(values, dtype=np.float64).ravel()
    L = lib()
    bits = np.array([L.oracle_f64_to_f16(float(t)) for t in v], dtype=np.uint16)
    return bits.view(np.float16).reshape(np.shape(values))


def f16_to_f64(values) -> np.ndarray:
    h = np.asarray(values, dtype=np.float16).view(np.uint16).ravel()
    L = lib()
    out = np.array([L.oracle_f16_to_f64(int(b)) for b in h], dtype=np.float64)
    return out.reshape(np.shape(values))


# ----------------------------------------------------------------------------- quantization

def quantize(x: np.ndarray, group_size: int = 0, qmax: int = 127):
    """Symmetric quantization of the rows of fp16 ``x [R, K]``.

    Returns ``(codes int8 [R, K], scales float32 [R] or [R, K/gs])``.
    ``group_size == 0`` gives one scale per row (per-token activations,
    per-output-channel weights)."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    R, K = x.shape
    q = np.empty((R, K), dtype=np.int8)
    G = 1 if group_size == 0 else K // group_size
    s = np.empty((R, G), dtype=np.float32)
    rc = lib().oracle_quantize_sym(_p(x.view(np.uint16), _u16p), R, K, group_size, qmax,
                                   _p(q, _i8p), _p(s, _f32p))
    if rc != 0:
        raise ValueError("oracle quantize: non-finite input or K not divisible by group size")
    return q, (s[:, 0].copy() if group_size == 0 else s)


def quantize_act(x: np.ndarray, group_size: int = 0):
    """Online per-token (or per-token-group) int8 activation quantization."""
    return quantize(x, group_size, 127)


def quantize_weight_int8(w: np.ndarray, group_size: int = 0):
    """Offline symmetric int8 weight quantization, per output channel or per group."""
    return quantize(w, group_size, 127)


def quantize_weight_int4(w: np.ndarray, group_size: int = 128):
    """Offline symmetric int4 per-group weight quantization: codes in [-7, 7]."""
    return quantize(w, group_size, 7)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    out = np.empty((N, K // 2), dtype=np.uint8)
    if lib().oracle_pack_int4(_p(codes, _i8p), N, K, _p(out, _u8p)) != 0:
        raise ValueError("K must be even")
    return out


def unpack_int4(packed: np.ndarray, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] * 2 == K
    out = np.empty((N, K), dtype=np.int8)
    lib().oracle_unpack_int4(_p(packed, _u8p), N, K, _p(out, _i8p))
    return out


def pack_weight_int4(w: np.ndarray, group_size: int = 128):
    """``(packed uint8 [N, K/2], scales float32 [N, K/gs])``."""
    codes, s = quantize_weight_int4(w, group_size)
    return pack_int4(codes), s


# ----------------------------------------------------------------------------- int8 GEMMs

def gemm_i32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """``C[m, n] = sum_k a[m, k] * b[n, k]`` in integers (int32 result)."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    c = np.empty((M, N), dtype=np.int32)
    if lib().oracle_gemm_i32(_p(a, _i8p), _p(b, _i8p), M, N, K, _p(c, _i32p)) != 0:
        raise OverflowError("int32 accumulator overflow")
    return c


def gemm_partials(a: np.ndarray, b: np.ndarray, group_size: int) -> np.ndarray:
    """Per-group partial sums ``P [G, M, N]``."""
    a = np.ascontiguousarray(a, dtype=np.int8)
    b = np.ascontiguousarray(b, dtype=np.int8)
    M, K = a.shape
    N = b.shape[0]
    G = K // group_size
    p = np.empty((G, M, N), dtype=np.int32)
    if lib().oracle_gemm_partials(_p(a, _i8p), _p(b, _i8p), M, N, K, group_size,
                                  _p(p, _i32p)) != 0:
        raise ValueError("K must be a multiple of the group size")
    return p


# ----------------------------------------------------------------------------- epilogues

def epilogue_pc(c: np.ndarray, sa: np.ndarray, sw: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.int32)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, N = c.shape
    y = np.empty((M, N), dtype=np.float16)
    lib().oracle_epilogue_pc(_p(c, _i32p), _p(sa, _f32p), _p(sw, _f32p), M, N,
                             _p(y.view(np.uint16), _u16p))
    return y


def epilogue_pg(p: np.ndarray, sa: np.ndarray, sw: np.ndarray):
    """Returns ``(y fp16 [M, N], T float64 [M, N])``."""
    p = np.ascontiguousarray(p, dtype=np.int32)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    G, M, N = p.shape
    assert sa.shape == (M, G) and sw.shape == (N, G)
    y = np.empty((M, N), dtype=np.float16)
    t = np.empty((M, N), dtype=np.float64)
    lib().oracle_epilogue_pg(_p(p, _i32p), _p(sa, _f32p), _p(sw, _f32p), M, N, G,
                             _p(y.view(np.uint16), _u16p), _p(t, _f64p))
    return y, t


def epilogue_w4a8(p: np.ndarray, sa: np.ndarray, sw: np.ndarray):
    """Returns ``(y fp16 [M, N], T float64 [M, N])``."""
    p = np.ascontiguousarray(p, dtype=np.int32)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    G, M, N = p.shape
    assert sa.shape == (M,) and sw.shape == (N, G)
    y = np.empty((M, N), dtype=np.float16)
    t = np.empty((M, N), dtype=np.float64)
    lib().oracle_epilogue_w4a8(_p(p, _i32p), _p(sa, _f32p), _p(sw, _f32p), M, N, G,
                               _p(y.view(np.uint16), _u16p), _p(t, _f64p))
    return y, t


# ----------------------------------------------------------------------------- whole layers

def w8a8_pc(x: np.ndarray, wq: np.ndarray, sw: np.ndarray) -> dict:
    """Per-channel W8A8: quantize x per token, int32 GEMM, rescale to fp16."""
    xq, sa = quantize_act(x, 0)
    c = gemm_i32(xq, wq)
    return dict(xq=xq, sa=sa, c=c, y=epilogue_pc(c, sa, sw))


def w8a8_pg(x: np.ndarray, wq: np.ndarray, sw: np.ndarray, group_size: int) -> dict:
    """Per-group W8A8: per-token-group activation scales, per-group partials."""
    xq, sa = quantize_act(x, group_size)
    p = gemm_partials(xq, wq, group_size)
    y, t = epilogue_pg(p, sa, sw)
    return dict(xq=xq, sa=sa, p=p, y=y, t=t)


def w4a8(x: np.ndarray, w4: np.ndarray, sw: np.ndarray, group_size: int) -> dict:
    """W4A8: per-token int8 activations against unpacked per-group int4 weights."""
    K = x.shape[1]
    xq, sa = quantize_act(x, 0)
    p = gemm_partials(xq, unpack_int4(w4, K), group_size)
    y, t = epilogue_w4a8(p, sa, sw)
    return dict(xq=xq, sa=sa, p=p, y=y, t=t)


def int8_mv(x: np.ndarray, wq: np.ndarray, sw: np.ndarray) -> dict:
    """Decode (M == 1): the same per-channel W8A8 pipeline on a single token."""
    x = np.asarray(x, dtype=np.float16).reshape(1, -1)
    return w8a8_pc(x, wq, sw)


def linear(mode: str, x: np.ndarray, w: np.ndarray, sw: np.ndarray, group_size: int = 0) -> dict:
    """Path selection: M == 1 in per-channel mode takes the matrix-vector path,
    everything else quantizes the activations and runs the mode's GEMM."""
    M = x.shape[0]
    if mode == "pc":
        return int8_mv(x, w, sw) if M == 1 else w8a8_pc(x, w, sw)
    if mode == "pg":
        return w8a8_pg(x, w, sw, group_size)
    if mode == "w4a8":
        return w4a8(x, w, sw, group_size)
    raise ValueError(mode)


# ----------------------------------------------------------------------------- comparison path

def w8a16(x: np.ndarray, wq: np.ndarray, sw: np.ndarray):
    """Weight-only int8 product (the pages' W8A16 baseline): returns
    ``(y fp16 [M, N], T float64 [M, N])`` with ``y = fp16(sw[n] * sum_k x w)``."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = x.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and sw.shape == (N,)
    y = np.empty((M, N), dtype=np.float16)
    t = np.empty((M, N), dtype=np.float64)
    lib().oracle_w8a16(_p(x.view(np.uint16), _u16p), _p(wq, _i8p), _p(sw, _f32p), M, N, K,
                       _p(y.view(np.uint16), _u16p), _p(t, _f64p))
    return y, t


def w4a16(x: np.ndarray, w4: np.ndarray, sw: np.ndarray, group_size: int):
    """Weight-only int4 product (the pages' W4A16 baseline): each code is
    dequantized to fp16(fl32(code * sw[n, g])); returns ``(y fp16 [M, N],
    T float64 [M, N])`` with ``y = fp16(sum_k x * w)``."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    M, K = x.shape
    codes = np.ascontiguousarray(unpack_int4(w4, K), dtype=np.int8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    N = codes.shape[0]
    assert sw.shape == (N, K // group_size)
    y = np.empty((M, N), dtype=np.float16)
    t = np.empty((M, N), dtype=np.float64)
    lib().oracle_w4a16(_p(x.view(np.uint16), _u16p), _p(codes, _i8p), _p(sw, _f32p), M, N, K,
                       group_size, _p(y.view(np.uint16), _u16p), _p(t, _f64p))
    return y, t
