"""GPU parity at the benchmark workloads' full sizes, through linear() (the
launch configuration the benchmark times).

Every output is compared, not a sample:

* activation and weight quantization: codes and scales in full, bit for bit;
* the layer's fp16 output: every element against the oracle within the fp16
  tolerance (per-channel) or the tolerance plus the per-group summation
  allowance; the oracle runs in bands of whole rows (per-token and per-group
  quantization and the GEMM are row-local, so a band of rows is the same
  sub-problem on both sides);
* per-channel: every int32 sum of the same GEMM kernel (the raw-sum export runs
  the product's tile configuration, asserted below), bit for bit;
* per-group and W4A8: the int32 partial sums of the full-size launch (the
  export takes the product's tile configuration, asserted) on whole-row bands
  covering every column -- the first and the last tile row -- bit for bit.

The oracle needs about a minute of host time for all shapes together on the
GPU machine's cores.
"""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, assert_fp16_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu

CASES = []
for name, wl in synth.WORKLOADS.items():
    for (M, N, K) in wl["shapes"]:
        CASES.append(pytest.param(wl["mode"], M, N, K, wl["gs"], wl["outliers"],
                                  id=f"{name}-{M}x{N}x{K}"))

# rows of int32 partials (G x rows x N x 4 bytes) the oracle holds at a time
_BAND_BYTES = 1 << 29


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


def _shape(cfg):
    """The tile configuration proper (occupancy may differ between the builds
    of one tile for different epilogues)."""
    return cfg["bm"], cfg["bn"], cfg["waves"]


def _bands(M, rows):
    return [(a, min(M, a + rows)) for a in range(0, M, rows)]


@pytest.mark.parametrize("mode,M,N,K,gs,outliers", CASES)
def test_workload_full_size(torch_gpu, oracle, mode, M, N, K, gs, outliers):
    import torch
    import w4a8_int8_gemm_amd as w
    print(f"workload mode={mode} M={M} N={N} K={K} gs={gs}", flush=True)
    x = synth.activations(M, K, seed=0, outliers=outliers)
    wt = synth.weights(N, K, seed=0)
    xd, wd = dev(x), dev(wt)

    # weights: the library's own offline quantizer, checked in full
    if mode == "w4a8":
        wg, swg = w.pack_weight_int4(wd, gs)
        wo, swo = oracle.pack_weight_int4(wt, gs)
        wcodes = oracle.unpack_int4(wo, K)
    else:
        wg, swg = w.quantize_weight_int8(wd, gs if mode == "pg" else 0)
        wo, swo = oracle.quantize_weight_int8(wt, gs if mode == "pg" else 0)
        wcodes = wo
    assert_equal(host(swg), swo, "weight scales")
    assert_equal(host(wg), wo, "weight codes")
    del wd

    # activations, checked in full
    act_gs = gs if mode == "pg" else 0
    xq, xs = w.quantize_act(xd, act_gs)
    xo, xso = oracle.quantize_act(x, act_gs)
    assert_equal(host(xs), xso, "activation scales")
    assert_equal(host(xq), xo, "activation codes")

    # the layer through linear(), every output
    y = host(w.linear({"pc": w.Mode.W8A8_PC, "pg": w.Mode.W8A8_PG, "w4a8": w.Mode.W4A8}[mode],
                      xd, wg, swg, gs))
    del xd
    if mode == "pc":
        c = host(w.w8a8_gemm_i32(xq, wg)) if M > 1 else None
        if M > 1:
            tile = _shape(w.gemm_tile_config(w.GemmOp.GEMM_PC, M, N, K))
            assert tile == _shape(w.gemm_tile_config(w.GemmOp.GEMM_I32, M, N, K)), tile
        for a, b in _bands(M, 512):
            c_ref = oracle.gemm_i32(xo[a:b], wcodes)
            if c is not None:
                assert_equal(c[a:b], c_ref, f"int32 sums, rows {a}..{b}")
            y_ref = oracle.epilogue_pc(c_ref, xso[a:b], swo)
            assert_fp16_close(y[a:b], y_ref, what=f"fp16 y, rows {a}..{b}")
        return

    G = K // gs
    epi = oracle.epilogue_pg if mode == "pg" else oracle.epilogue_w4a8
    rows = max(1, min(512, _BAND_BYTES // (G * N * 4)))
    for a, b in _bands(M, rows):
        p_ref = oracle.gemm_partials(xo[a:b], wcodes, gs)
        y_ref, t = epi(p_ref, xso[a:b], swo)
        assert_fp16_close(y[a:b], y_ref, t, G, what=f"fp16 y, rows {a}..{b}")
    del y

    # int32 partials of the full-size launch, first and last tile rows
    prod = w.GemmOp.GEMM_PG if mode == "pg" else w.GemmOp.GEMM_W4A8
    part = w.GemmOp.PG_PARTIALS if mode == "pg" else w.GemmOp.W4A8_PARTIALS
    tp = _shape(w.gemm_tile_config(part, M, N, K, gs))
    assert tp == _shape(w.gemm_tile_config(prod, M, N, K, gs)), tp
    bm = tp[0]
    p = (w.w8a8_gemm_pg_partials(xq, wg, gs) if mode == "pg"
         else w.w4a8_gemm_partials(xq, wg, gs))
    last = ((M - 1) // bm) * bm
    for a, b in ((0, bm), (last, M)):
        got = host(p[:, a:b, :].contiguous())
        assert_equal(got, oracle.gemm_partials(xo[a:b], wcodes, gs),
                     f"int32 partials, tile rows {a}..{b}")
    del p
    torch.cuda.empty_cache()
