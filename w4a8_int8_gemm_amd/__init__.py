"""MI355X (gfx950) W8A8 / W4A8 int8 linear layer -- Python binding.

Thin wrappers with the C ABI's names (include/w4a8.h): they check tensors,
allocate outputs with torch, and pass device pointers and torch's current
HIP stream to libw4a8.so.  Every step of the computation runs in the
library's HIP kernels; nothing here computes.

    xq, xs = quantize_act(x)                      # fp16 [M, K] -> int8, fp32 [M]
    wq, sw = quantize_weight_int8(w)               # offline, per output channel
    y = w8a8_gemm_pc(xq, xs, wq, sw)               # fp16 [M, N]
    y = linear(Mode.W8A8_PC, x, wq, sw)            # the whole layer, MV when M == 1
    y = w8a8_mv_pg(x1, wq, sw, 128)                # decode with per-group scales
"""
from __future__ import annotations

from ._lib import LIB_PATH, GemmOp, Mode, Status, W4A8Error, check, lib
from .ops import (gemm_tile_config, int8_mv, is_available, linear, linear_noalloc,
                  linear_workspace_size, pack_weight_int4,
                  quantize_act, quantize_weight_int8, w4a8_gemm, w4a8_gemm_partials,
                  w4a8_mv, w8a8_gemm_i32, w8a8_gemm_pc, w8a8_gemm_pg, w8a8_gemm_pg_partials,
                  w8a8_mv_pg, w8a16_gemm, w4a16_gemm)

__all__ = [
    "LIB_PATH", "GemmOp", "Mode", "Status", "gemm_tile_config", "W4A8Error", "check", "lib", "int8_mv", "is_available",
    "linear", "linear_noalloc", "linear_workspace_size", "pack_weight_int4", "quantize_act",
    "quantize_weight_int8", "w4a8_gemm", "w4a8_gemm_partials", "w8a8_gemm_i32",
    "w8a8_gemm_pc", "w8a8_gemm_pg", "w8a8_gemm_pg_partials", "w4a8_mv", "w8a8_mv_pg",
    "w8a16_gemm", "w4a16_gemm",
]
