"""GPU parity of the weight-only int8 comparison GEMM (w8a16_gemm) against
the oracle: fp16 outputs within 2e-3 relative (floor 2^-14) plus the fp32
accumulation bound gamma_K * T, ragged edges and the pages' N=10240, K=2560
shape (sampled rows at M=4096)."""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_fp16_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


SHAPES = [(16, 512, 256), (3, 100, 384), (257, 321, 512), (200, 302, 640), (130, 1000, 64),
          (1024, 4096, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a16_small(torch_gpu, oracle, M, N, K):
    import w4a8_int8_gemm_amd as w
    print(f"w8a16 M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, seed=M + N)
    wq, sw = oracle.quantize_weight_int8(synth.weights(N, K, seed=K), 0)
    y_ref, t_ref = oracle.w8a16(x, wq, sw)
    y = w.w8a16_gemm(dev(x), dev(wq), dev(sw))
    stats = assert_fp16_close(host(y), y_ref, t_ref, K - 2, what="w8a16 y")
    assert stats["exact_frac"] > 0.9, stats


def test_w8a16_pages_shape_sampled(torch_gpu, oracle):
    import w4a8_int8_gemm_amd as w
    M, N, K = 4096, 10240, 2560
    print(f"w8a16 M={M} N={N} K={K} (sampled rows)", flush=True)
    x = synth.activations(M, K, seed=0)
    wq, sw = oracle.quantize_weight_int8(synth.weights(N, K, seed=0), 0)
    y = host(w.w8a16_gemm(dev(x), dev(wq), dev(sw)))
    rows = synth.sample_indices(M, 24, seed=7, salt=3)
    y_ref, t_ref = oracle.w8a16(x[rows], wq, sw)
    stats = assert_fp16_close(y[rows], y_ref, t_ref, K - 2, what="w8a16 y (sampled rows)")
    assert stats["exact_frac"] > 0.9, stats


def test_w8a16_empty_and_bad_args(torch_gpu):
    import torch
    import w4a8_int8_gemm_amd as w
    x = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    wq = torch.zeros((8, 64), dtype=torch.int8, device="cuda")
    sw = torch.ones(8, dtype=torch.float32, device="cuda")
    assert w.w8a16_gemm(x, wq, sw).shape == (0, 8)
    with pytest.raises(Exception):
        w.w8a16_gemm(torch.zeros((4, 40), dtype=torch.float16, device="cuda"),
                     torch.zeros((8, 40), dtype=torch.int8, device="cuda"), sw)


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", [(16, 512, 256), (3, 100, 384), (257, 321, 512), (200, 302, 640),
                                   (1024, 4096, 256)])
def test_w4a16_small(torch_gpu, oracle, M, N, K, gs):
    import w4a8_int8_gemm_amd as w
    if K % gs:
        pytest.skip("K not a multiple of gs")
    print(f"w4a16 M={M} N={N} K={K} gs={gs}", flush=True)
    x = synth.activations(M, K, seed=M + N)
    w4, s4 = oracle.pack_weight_int4(synth.weights(N, K, seed=K), gs)
    y_ref, t_ref = oracle.w4a16(x, w4, s4, gs)
    y = w.w4a16_gemm(dev(x), dev(w4), dev(s4), gs)
    stats = assert_fp16_close(host(y), y_ref, t_ref, K - 2, what="w4a16 y")
    assert stats["exact_frac"] > 0.9, stats


def test_w4a16_every_nibble(torch_gpu, oracle):
    """Packed bytes covering every nibble, including 0x8 (code -8)."""
    import w4a8_int8_gemm_amd as w
    M, N, K, gs = 64, 256, 256, 128
    x = synth.activations(M, K, seed=9)
    w4 = synth.packed_int4(N, K, 9, 1)
    s4 = synth.scales(N, K // gs, 9, 1, 0.3)
    y_ref, t_ref = oracle.w4a16(x, w4, s4, gs)
    y = w.w4a16_gemm(dev(x), dev(w4), dev(s4), gs)
    assert_fp16_close(host(y), y_ref, t_ref, K - 2, what="w4a16 y (every nibble)")


@pytest.mark.parametrize("N,K", [(10240, 2560), (333, 4096), (7, 16384), (130, 64)])
def test_weight_only_decode(torch_gpu, oracle, N, K):
    """M == 1 takes the matrix-vector form (K <= 16384); same oracle, same bound."""
    import w4a8_int8_gemm_amd as w
    print(f"weight-only decode N={N} K={K}", flush=True)
    x = synth.activations(1, K, seed=N)
    wt = synth.weights(N, K, seed=K)
    wq, sw = oracle.quantize_weight_int8(wt, 0)
    y_ref, t_ref = oracle.w8a16(x, wq, sw)
    y = w.w8a16_gemm(dev(x), dev(wq), dev(sw))
    assert_fp16_close(host(y), y_ref, t_ref, K - 2, what="w8a16 decode")
    w4, s4 = oracle.pack_weight_int4(wt, 64)
    y_ref, t_ref = oracle.w4a16(x, w4, s4, 64)
    y = w.w4a16_gemm(dev(x), dev(w4), dev(s4), 64)
    assert_fp16_close(host(y), y_ref, t_ref, K - 2, what="w4a16 decode")
