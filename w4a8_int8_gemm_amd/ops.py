"""torch-tensor wrappers over the C entry points (marshalling only).

Each function checks every tensor's dtype, device, contiguity and exact shape
(scales included: the C ABI receives bare pointers and cannot tell a short or
misplaced scale vector from a valid one), allocates missing outputs with
torch, and calls the library on torch's current stream of the tensors'
device.  Outputs may be passed in (``out=...``) to avoid allocations.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import GemmOp, Mode, check, lib


# Device type the wrappers accept (HIP devices appear as "cuda" in torch).
_DEVICE_TYPE = "cuda"


def _need(t, dtype, name, ndim, like=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != _DEVICE_TYPE:
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {like.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shaped(t, dtype, shape, name, like):
    """t must be a contiguous `dtype` tensor of exactly `shape` on like's device."""
    _need(t, dtype, name, len(shape), like)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _groups(K: int, group_size: int) -> int:
    """K / group_size for a per-group operation (group size 64 or 128 dividing K)."""
    if group_size not in (64, 128):
        raise ValueError(f"group_size must be 64 or 128, got {group_size}")
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    return K // group_size


def _out(t, shape, dtype, like, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _shaped(t, dtype, shape, name, like)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _st(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def is_available() -> bool:
    """True if the current HIP device is a gfx950 GPU."""
    return bool(lib().w4a8_is_available())


def _scale_shape(rows, K, group_size):
    return (rows,) if group_size == 0 else (rows, K // group_size if group_size > 0 else 0)


def quantize_act(x, group_size: int = 0, out=None, scale=None):
    """fp16 [M, K] -> (int8 [M, K], fp32 [M] or [M, K/gs])."""
    _need(x, torch.float16, "x", 2)
    M, K = x.shape
    out = _out(out, (M, K), torch.int8, x, "out")
    scale = _out(scale, _scale_shape(M, K, group_size), torch.float32, x, "scale")
    with torch.cuda.device(x.device):
        check(lib().quantize_act(_p(x), M, K, group_size, _p(out), _p(scale), _st(x)))
    return out, scale


def quantize_weight_int8(w, group_size: int = 0, out=None, scale=None):
    """fp16 [N, K] -> (int8 [N, K], fp32 [N] or [N, K/gs])."""
    _need(w, torch.float16, "w", 2)
    N, K = w.shape
    out = _out(out, (N, K), torch.int8, w, "out")
    scale = _out(scale, _scale_shape(N, K, group_size), torch.float32, w, "scale")
    with torch.cuda.device(w.device):
        check(lib().quantize_weight_int8(_p(w), N, K, group_size, _p(out), _p(scale), _st(w)))
    return out, scale


def pack_weight_int4(w, group_size: int = 128, out=None, scale=None):
    """fp16 [N, K] -> (packed uint8 [N, K/2], fp32 [N, K/gs])."""
    _need(w, torch.float16, "w", 2)
    N, K = w.shape
    out = _out(out, (N, K // 2), torch.uint8, w, "out")
    scale = _out(scale, (N, K // group_size if group_size > 0 else 0), torch.float32, w, "scale")
    with torch.cuda.device(w.device):
        check(lib().pack_weight_int4(_p(w), N, K, group_size, _p(out), _p(scale), _st(w)))
    return out, scale


def _gemm_shapes(xq, w, packed):
    _need(xq, torch.int8, "xq", 2)
    _need(w, torch.uint8 if packed else torch.int8, "w", 2, xq)
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] * (2 if packed else 1) != K:
        raise ValueError(f"weight shape {tuple(w.shape)} does not match K={K}")
    return M, N, K


def w8a8_gemm_pc(xq, x_scale, wq, w_scale, out=None):
    """y fp16 [M, N] = (xq . wq^T) * x_scale[m] * w_scale[n]."""
    M, N, K = _gemm_shapes(xq, wq, False)
    _shaped(x_scale, torch.float32, (M,), "x_scale", xq)
    _shaped(w_scale, torch.float32, (N,), "w_scale", xq)
    out = _out(out, (M, N), torch.float16, xq, "out")
    with torch.cuda.device(xq.device):
        check(lib().w8a8_gemm_pc(_p(xq), _p(x_scale), _p(wq), _p(w_scale), _p(out), M, N, K,
                                 _st(xq)))
    return out


def w8a8_gemm_pg(xq, x_scale, wq, w_scale, group_size: int, out=None):
    """Per-group W8A8: x_scale [M, K/gs], w_scale [N, K/gs]."""
    M, N, K = _gemm_shapes(xq, wq, False)
    G = _groups(K, group_size)
    _shaped(x_scale, torch.float32, (M, G), "x_scale", xq)
    _shaped(w_scale, torch.float32, (N, G), "w_scale", xq)
    out = _out(out, (M, N), torch.float16, xq, "out")
    with torch.cuda.device(xq.device):
        check(lib().w8a8_gemm_pg(_p(xq), _p(x_scale), _p(wq), _p(w_scale), group_size, _p(out),
                                 M, N, K, _st(xq)))
    return out


def w4a8_gemm(xq, x_scale, w4, w_scale, group_size: int, out=None):
    """W4A8: per-token x_scale [M], packed w4 [N, K/2], w_scale [N, K/gs]."""
    M, N, K = _gemm_shapes(xq, w4, True)
    G = _groups(K, group_size)
    _shaped(x_scale, torch.float32, (M,), "x_scale", xq)
    _shaped(w_scale, torch.float32, (N, G), "w_scale", xq)
    out = _out(out, (M, N), torch.float16, xq, "out")
    with torch.cuda.device(xq.device):
        check(lib().w4a8_gemm(_p(xq), _p(x_scale), _p(w4), _p(w_scale), group_size, _p(out),
                              M, N, K, _st(xq)))
    return out


def int8_mv(x, wq, w_scale, out=None, return_codes: bool = False):
    """Decode: x fp16 [K] (or [1, K]) -> y fp16 [N]; optionally also (codes, scale)."""
    if x.dim() == 2 and x.shape[0] == 1:
        x = x.reshape(-1)
    _need(x, torch.float16, "x", 1)
    _need(wq, torch.int8, "wq", 2, x)
    K = x.shape[0]
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("wq does not match K")
    _shaped(w_scale, torch.float32, (N,), "w_scale", x)
    out = _out(out, (N,), torch.float16, x, "out")
    xq = torch.empty((K,), dtype=torch.int8, device=x.device) if return_codes else None
    xs = torch.empty((1,), dtype=torch.float32, device=x.device) if return_codes else None
    with torch.cuda.device(x.device):
        check(lib().int8_mv(_p(x), _p(wq), _p(w_scale), _p(out), N, K, _p(xq), _p(xs), _st(x)))
    return (out, xq, xs) if return_codes else out


def _mv_group(fn, x, w, w_scale, group_size: int, packed: bool, out):
    if x.dim() == 2 and x.shape[0] == 1:
        x = x.reshape(-1)
    _need(x, torch.float16, "x", 1)
    _need(w, torch.uint8 if packed else torch.int8, "w", 2, x)
    K = x.shape[0]
    N = w.shape[0]
    if w.shape[1] * (2 if packed else 1) != K:
        raise ValueError("weight shape does not match K")
    _shaped(w_scale, torch.float32, (N, _groups(K, group_size)), "w_scale", x)
    out = _out(out, (N,), torch.float16, x, "out")
    with torch.cuda.device(x.device):
        check(getattr(lib(), fn)(_p(x), _p(w), _p(w_scale), group_size, _p(out), N, K, _st(x)))
    return out


def w8a8_mv_pg(x, wq, w_scale, group_size: int, out=None):
    """Decode, per-group W8A8: x fp16 [K] -> y fp16 [N]; w_scale [N, K/gs]."""
    return _mv_group("w8a8_mv_pg", x, wq, w_scale, group_size, False, out)


def w4a8_mv(x, w4, w_scale, group_size: int, out=None):
    """Decode, W4A8: x fp16 [K], packed w4 [N, K/2], w_scale [N, K/gs] -> y fp16 [N]."""
    return _mv_group("w4a8_mv", x, w4, w_scale, group_size, True, out)


def linear_workspace_size(mode, M: int, K: int, group_size: int = 0) -> int:
    return int(lib().linear_workspace_size(int(mode), M, K, group_size))


def linear(mode, x, w, w_scale, group_size: int = 0, workspace=None, out=None):
    """The whole layer: the mode's matrix-vector kernel when M == 1, else quantize + GEMM."""
    mode = Mode(mode)
    _need(x, torch.float16, "x", 2)
    packed = mode == Mode.W4A8
    _need(w, torch.uint8 if packed else torch.int8, "w", 2, x)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] * (2 if packed else 1) != K:
        raise ValueError("weight shape does not match K")
    sw_shape = (N,) if mode == Mode.W8A8_PC else (N, _groups(K, group_size))
    _shaped(w_scale, torch.float32, sw_shape, "w_scale", x)
    need = linear_workspace_size(mode, M, K, group_size)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    else:
        _need(workspace, torch.uint8, "workspace", 1, x)
        if workspace.numel() < need:
            raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    out = _out(out, (M, N), torch.float16, x, "out")
    with torch.cuda.device(x.device):
        check(lib().linear(int(mode), _p(x), M, K, _p(w), _p(w_scale), group_size, N, _p(out),
                           _p(workspace), workspace.numel(), _st(x)))
    return out


def linear_noalloc(mode, x, w, w_scale, group_size: int = 0, out=None):
    """linear() without a workspace: the library keeps the activation codes in
    a static 64 MiB device array (no allocation in the call; calls that overlap
    on one GPU race).  Pass ``out`` to keep this wrapper allocation-free too."""
    mode = Mode(mode)
    _need(x, torch.float16, "x", 2)
    packed = mode == Mode.W4A8
    _need(w, torch.uint8 if packed else torch.int8, "w", 2, x)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] * (2 if packed else 1) != K:
        raise ValueError("weight shape does not match K")
    sw_shape = (N,) if mode == Mode.W8A8_PC else (N, _groups(K, group_size))
    _shaped(w_scale, torch.float32, sw_shape, "w_scale", x)
    out = _out(out, (M, N), torch.float16, x, "out")
    with torch.cuda.device(x.device):
        check(lib().linear_noalloc(int(mode), _p(x), M, K, _p(w), _p(w_scale), group_size, N,
                                   _p(out), _st(x)))
    return out


def w8a8_gemm_i32(xq, wq, out=None):
    """Raw int32 sums [M, N] of the per-channel GEMM's main loop."""
    M, N, K = _gemm_shapes(xq, wq, False)
    out = _out(out, (M, N), torch.int32, xq, "out")
    with torch.cuda.device(xq.device):
        check(lib().w8a8_gemm_i32(_p(xq), _p(wq), _p(out), M, N, K, _st(xq)))
    return out


def w8a8_gemm_pg_partials(xq, wq, group_size: int, out=None):
    """Per-group int32 partial sums [K/gs, M, N]."""
    M, N, K = _gemm_shapes(xq, wq, False)
    out = _out(out, (_groups(K, group_size), M, N), torch.int32, xq, "out")
    with torch.cuda.device(xq.device):
        check(lib().w8a8_gemm_pg_partials(_p(xq), _p(wq), group_size, _p(out), M, N, K, _st(xq)))
    return out


def w4a8_gemm_partials(xq, w4, group_size: int, out=None):
    """Per-group int32 partial sums [K/gs, M, N] against unpacked int4 codes."""
    M, N, K = _gemm_shapes(xq, w4, True)
    out = _out(out, (_groups(K, group_size), M, N), torch.int32, xq, "out")
    with torch.cuda.device(xq.device):
        check(lib().w4a8_gemm_partials(_p(xq), _p(w4), group_size, _p(out), M, N, K, _st(xq)))
    return out


def w8a16_gemm(x, wq, w_scale, out=None):
    """Weight-only int8 comparison GEMM: y fp16 [M, N] = w_scale[n] * (x . wq^T),
    x fp16 [M, K] (not quantized), wq int8 [N, K], w_scale fp32 [N]."""
    _need(x, torch.float16, "x", 2)
    _need(wq, torch.int8, "wq", 2, x)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError(f"weight shape {tuple(wq.shape)} does not match K={K}")
    _shaped(w_scale, torch.float32, (N,), "w_scale", x)
    out = _out(out, (M, N), torch.float16, x, "out")
    with torch.cuda.device(x.device):
        check(lib().w8a16_gemm(_p(x), _p(wq), _p(w_scale), _p(out), M, N, K, _st(x)))
    return out


def w4a16_gemm(x, w4, w_scale, group_size: int, out=None):
    """Weight-only int4 comparison GEMM: y fp16 [M, N] = sum_k x[m,k] *
    fp16(code[n,k] * w_scale[n, k // gs]); x fp16 [M, K], w4 uint8 [N, K/2],
    w_scale fp32 [N, K/gs] (as from pack_weight_int4)."""
    _need(x, torch.float16, "x", 2)
    _need(w4, torch.uint8, "w4", 2, x)
    M, K = x.shape
    N = w4.shape[0]
    if w4.shape[1] * 2 != K:
        raise ValueError(f"weight shape {tuple(w4.shape)} does not match K={K}")
    _shaped(w_scale, torch.float32, (N, _groups(K, group_size)), "w_scale", x)
    out = _out(out, (M, N), torch.float16, x, "out")
    with torch.cuda.device(x.device):
        check(lib().w4a16_gemm(_p(x), _p(w4), _p(w_scale), group_size, _p(out), M, N, K, _st(x)))
    return out


def gemm_tile_config(op, M: int, N: int, K: int, group_size: int = 0) -> dict:
    """The kernel configuration a GEMM entry point runs for these sizes on the
    current device (nothing is launched): tile rows and columns (bm == 0: the
    few-token matrix-vector form), waves per workgroup, workgroups launched,
    output tiles and workgroups per compute unit."""
    out = (ctypes.c_int64 * 6)()
    check(lib().gemm_tile_config(int(GemmOp(op)), M, N, K, group_size, out))
    return dict(bm=out[0], bn=out[1], waves=out[2], grid=out[3], tiles=out[4], per_cu=out[5])
