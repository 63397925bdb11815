"""Helpers shared by the GPU parity tests: device transfer, the fp16
tolerance, sampled oracle evaluation at full size, and readable reports."""
from __future__ import annotations

import numpy as np
import pytest

U = 2.0 ** -24          # unit roundoff of fp32
REL = 2e-3              # relative bound on fp16 outputs
FLOOR = 2.0 ** -14      # smallest normal fp16: relative bound floor for tiny outputs


def gamma(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32 (recursive summation bound)."""
    return n * U / (1.0 - n * U)


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w4a8_int8_gemm_amd as w
    if not w.is_available():
        pytest.fail("a GPU is present but it is not gfx950: " + w.lib().w4a8_last_error().decode())
    return torch


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_fp16_close(y: np.ndarray, ref: np.ndarray, T: np.ndarray | None = None, G: int = 0,
                      what: str = ""):
    """|y - ref| <= 2e-3 * max(|ref|, 2^-14) [+ gamma_{G+2} * T for grouped sums]."""
    y64 = y.astype(np.float64)
    r64 = ref.astype(np.float64)
    assert np.all(np.isfinite(y64)), f"{what}: non-finite output"
    err = np.abs(y64 - r64)
    bound = REL * np.maximum(np.abs(r64), FLOOR)
    if T is not None:
        bound = bound + gamma(G + 2) * T
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {y64[tuple(i)]!r} want {r64[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs out of tolerance; {detail}")
    rel = err / np.maximum(np.abs(r64), FLOOR)
    return dict(max_rel=float(rel.max()) if rel.size else 0.0,
                n_over_strict=int((rel > REL).sum()),
                exact_frac=float((y64 == r64).mean()) if y64.size else 1.0)


def assert_equal(got: np.ndarray, want: np.ndarray, what: str):
    if got.shape != want.shape:
        raise AssertionError(f"{what}: shape {got.shape} != {want.shape}")
    neq = got != want
    if neq.any():
        idx = np.argwhere(neq)[:5]
        detail = ", ".join(f"{tuple(i)}: got {got[tuple(i)]!r} want {want[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(neq.sum())} of {neq.size} differ; {detail}")
