"""Seeded synthetic inputs shared by the CPU oracle, the GPU tests and the benchmark.

This module only draws random numbers and shapes them; it holds none of the
quantization or GEMM arithmetic, so neither the oracle nor the HIP path depends
on the other through it.

Workloads (fp16 sources, row-major, K contiguous):

* activations ``X [M, K]``: standard normal, optionally with outlier channels
  (x50) and outlier tokens (x20) applied in fp32 before the cast to fp16, the
  stress case for per-token scales;
* weights ``W [N, K]``: normal with sigma 0.02.

The shapes stand in for the pages' single-operator table (N=10240, K=2560,
"cider" post, section on performance measurements), the 4516-token prefill
context (Apple-silicon essay, section on MLX and the prefill bottleneck) and an
8B-class decoder layer; all weights are random-init.
"""
from __future__ import annotations

import numpy as np

# Stream ids keep activations, weights and outlier picks independent of each other.
_STREAM_X = 1
_STREAM_W = 2
_STREAM_OUTLIER = 3


def activations(M: int, K: int, seed: int = 0, outliers: bool = False) -> np.ndarray:
    """fp16 ``[M, K]`` drawn N(0, 1); with ``outliers`` 8 channels x50 and 1 % of tokens x20."""
    rng = np.random.default_rng([seed, _STREAM_X])
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        ro = np.random.default_rng([seed, _STREAM_OUTLIER])
        chans = ro.choice(K, size=min(8, K), replace=False)
        x[:, chans] *= 50.0
        ntok = int(round(0.01 * M))
        if ntok > 0:
            toks = ro.choice(M, size=ntok, replace=False)
            x[toks, :] *= 20.0
    return x.astype(np.float16)


def weights(N: int, K: int, seed: int = 0, layer: int = 0, sigma: float = 0.02) -> np.ndarray:
    """fp16 ``[N, K]`` drawn N(0, sigma^2); ``layer`` selects an independent stream."""
    rng = np.random.default_rng([seed, _STREAM_W, layer])
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    return w.astype(np.float16)


def int8_codes(rows: int, K: int, seed: int = 0, salt: int = 0) -> np.ndarray:
    """int8 ``[rows, K]`` in [-127, 127], bell-shaped like quantized normal data,
    with the extreme codes present in every row."""
    rng = np.random.default_rng([seed, 4, salt])
    c = np.clip(np.rint(rng.standard_normal((rows, K)) * 42.0), -127, 127).astype(np.int8)
    if K >= 2:
        c[:, rng.integers(0, K)] = 127
        c[:, rng.integers(0, K)] = -127
    return c


def packed_int4(rows: int, K: int, seed: int = 0, salt: int = 0) -> np.ndarray:
    """uint8 ``[rows, K/2]``: random bytes, i.e. every nibble value including 0x8."""
    rng = np.random.default_rng([seed, 5, salt])
    return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


def scales(rows: int, groups: int = 0, seed: int = 0, salt: int = 0, magnitude: float = 0.02) -> np.ndarray:
    """Positive fp32 scales ``[rows]`` (groups == 0) or ``[rows, groups]``."""
    rng = np.random.default_rng([seed, 6, salt])
    shape = (rows,) if groups == 0 else (rows, groups)
    return (rng.uniform(0.25, 4.0, size=shape) * magnitude / 127.0).astype(np.float32)


def sample_indices(n: int, count: int, seed: int = 0, salt: int = 0) -> np.ndarray:
    """Sorted distinct indices in ``[0, n)`` that always include the first and last index."""
    rng = np.random.default_rng([seed, 7, salt])
    count = min(count, n)
    picks = set(rng.choice(n, size=count, replace=False).tolist())
    picks.update({0, n - 1})
    return np.array(sorted(picks), dtype=np.int64)


# Named workloads.  Each entry: mode, shapes, group size, outliers.
WORKLOADS = {
    # tiny per-channel case, small enough for exhaustive oracle checks
    "pc_tiny": dict(mode="pc", shapes=[(16, 512, 256)], gs=0, outliers=False),
    # per-channel M sweep at N=10240, K=2560 (M=1 is the decode matrix-vector path)
    "pc_sweep": dict(mode="pc", shapes=[(1, 10240, 2560), (128, 10240, 2560), (1024, 10240, 2560)],
                     gs=0, outliers=False),
    # large prefill with outlier channels and tokens
    "pc_large": dict(mode="pc", shapes=[(4096, 10240, 2560), (8192, 10240, 2560)], gs=0, outliers=True),
    # per-group, both operands scaled per group of gs along K
    "pg_gs128": dict(mode="pg", shapes=[(4096, 4096, 4096), (4096, 14336, 4096), (4096, 4096, 14336)],
                     gs=128, outliers=False),
    "pg_gs64": dict(mode="pg", shapes=[(4096, 4096, 4096), (4096, 14336, 4096), (4096, 4096, 14336)],
                    gs=64, outliers=False),
    # int4 weights, decoder-layer linears at a 4516-token prefill (qkv, o, gate_up, down)
    "w4a8_layer": dict(mode="w4a8", shapes=[(4516, 6144, 4096), (4516, 4096, 4096),
                                            (4516, 24576, 4096), (4516, 4096, 12288)],
                       gs=128, outliers=False),
    # one GPU's share when a layer's output columns are split over eight GPUs:
    # the headline layer (N = 10240 / 8) and the W4A8 gate_up linear (24576 / 8)
    "pc_shard8": dict(mode="pc", shapes=[(4096, 1280, 2560)], gs=0, outliers=True),
    "w4a8_shard8": dict(mode="w4a8", shapes=[(4516, 3072, 4096)], gs=128, outliers=False),
}

# The headline shape: per-channel W8A8 prefill at M=4096, N=10240, K=2560.
HEADLINE = dict(workload="pc_large", M=4096, N=10240, K=2560, outliers=True)
