"""GPU parity at the benchmark workloads' full sizes, through linear() (the
launch configuration the benchmark times).

Activation and weight quantization are compared in full, bit for bit.  The
fp16 outputs are compared on a sample of rows x columns that the oracle
computes on the sampled sub-problem (per-token and per-channel/per-group
quantization are row-local, so the sub-problem's codes are the full
problem's codes); the per-channel int32 sums are compared on the same sample.
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


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


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

    # the layer through linear()
    m_idx = synth.sample_indices(M, 48, seed=M, salt=1)
    n_idx = synth.sample_indices(N, 256, seed=N, salt=2)
    y = w.linear({"pc": w.Mode.W8A8_PC, "pg": w.Mode.W8A8_PG, "w4a8": w.Mode.W4A8}[mode],
                 xd, wg, swg, gs)
    ys = host(y[torch.as_tensor(m_idx, device="cuda")][:, torch.as_tensor(n_idx, device="cuda")])
    del y

    xs_sub, ws_sub = xo[m_idx], wcodes[n_idx]
    if mode == "pc":
        c = oracle.gemm_i32(xs_sub, ws_sub)
        y_ref = oracle.epilogue_pc(c, xso[m_idx], swo[n_idx])
        assert_fp16_close(ys, y_ref, what="fp16 y (sample)")
        if M > 1:
            cg = w.w8a8_gemm_i32(xq, wg)
            cs = host(cg[torch.as_tensor(m_idx, device="cuda")][:, torch.as_tensor(n_idx, device="cuda")])
            assert_equal(cs, c, "int32 sums (sample)")
    elif mode == "pg":
        p = oracle.gemm_partials(xs_sub, ws_sub, gs)
        y_ref, t = oracle.epilogue_pg(p, xso[m_idx], swo[n_idx])
        assert_fp16_close(ys, y_ref, t, K // gs, what="fp16 y (sample)")
    else:
        p = oracle.gemm_partials(xs_sub, ws_sub, gs)
        y_ref, t = oracle.epilogue_w4a8(p, xso[m_idx], swo[n_idx])
        assert_fp16_close(ys, y_ref, t, K // gs, what="fp16 y (sample)")
    torch.cuda.empty_cache()
