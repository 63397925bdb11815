"""GPU parity of the decode matrix-vector kernel and of linear()'s path
selection, each side running its own whole pipeline from the fp16 sources."""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, assert_fp16_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


@pytest.mark.parametrize("N,K", [(10240, 2560), (512, 256), (100, 16), (333, 4096),
                                 (64, 14336), (257, 4112), (7, 32768)])
def test_int8_mv(torch_gpu, oracle, N, K):
    import w4a8_int8_gemm_amd as w
    print(f"int8_mv N={N} K={K}", flush=True)
    x = synth.activations(1, K, seed=K, outliers=True)
    wt = synth.weights(N, K, seed=N)
    wq, sw = oracle.quantize_weight_int8(wt)
    r = oracle.int8_mv(x, wq, sw)
    y, xq, xs = w.int8_mv(dev(x[0]), dev(wq), dev(sw), return_codes=True)
    assert_equal(host(xs), r["sa"], "token scale")
    assert_equal(host(xq), r["xq"][0], "token codes")
    assert_fp16_close(host(y), r["y"][0], what="fp16 y")
    # bit-identical to quantize_act + w8a8_gemm_pc at M = 1 (where the GEMM
    # accepts K), which runs the few-token form there; the comparison with
    # the tiled GEMM itself is in test_gpu_few_token.py
    if K % 64 == 0:
        xq2, xs2 = w.quantize_act(dev(x))
        y2 = w.w8a8_gemm_pc(xq2, xs2, dev(wq), dev(sw))
        assert_equal(host(y), host(y2)[0], "MV vs w8a8_gemm_pc at M=1")


def test_int8_mv_zero_token(torch_gpu, oracle):
    import w4a8_int8_gemm_amd as w
    x = np.zeros((2560,), np.float16)
    wq, sw = oracle.quantize_weight_int8(synth.weights(64, 2560))
    y, xq, xs = w.int8_mv(dev(x), dev(wq), dev(sw), return_codes=True)
    assert np.all(host(y) == 0) and np.all(host(xq) == 0) and host(xs)[0] == 0


@pytest.mark.parametrize("M", [1, 2, 4, 5, 64, 300])
def test_linear_pc_end_to_end(torch_gpu, oracle, M):
    """GPU: quantize_weight_int8 + linear.  Oracle: its own quantizer + GEMM."""
    import w4a8_int8_gemm_amd as w
    N, K = 384, 512
    x = synth.activations(M, K, seed=M, outliers=True)
    wt = synth.weights(N, K, seed=7)
    wq_g, sw_g = w.quantize_weight_int8(dev(wt))
    wq, sw = oracle.quantize_weight_int8(wt)
    assert_equal(host(wq_g), wq, "weight codes")
    assert_equal(host(sw_g), sw, "weight scales")
    r = oracle.linear("pc", x, wq, sw)
    y = w.linear(w.Mode.W8A8_PC, dev(x), wq_g, sw_g)
    assert_fp16_close(host(y), r["y"], what=f"linear pc M={M}")
    if M == 1:   # the dispatch picked the MV kernel: identical to calling it directly
        assert_equal(host(y)[0], host(w.int8_mv(dev(x[0]), wq_g, sw_g)), "dispatch to MV")
    else:        # identical to quantize_act + w8a8_gemm_pc (few-token form at M <= 4)
        xq, xs = w.quantize_act(dev(x))
        assert_equal(host(y), host(w.w8a8_gemm_pc(xq, xs, wq_g, sw_g)),
                     "dispatch to quantize_act + w8a8_gemm_pc")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M", [1, 3, 130])
def test_linear_pg_end_to_end(torch_gpu, oracle, M, gs):
    import w4a8_int8_gemm_amd as w
    N, K = 200, 1024
    x = synth.activations(M, K, seed=M + gs, outliers=True)
    wt = synth.weights(N, K, seed=8)
    wq_g, sw_g = w.quantize_weight_int8(dev(wt), gs)
    wq, sw = oracle.quantize_weight_int8(wt, gs)
    assert_equal(host(wq_g), wq, "weight codes")
    r = oracle.linear("pg", x, wq, sw, gs)
    y = w.linear(w.Mode.W8A8_PG, dev(x), wq_g, sw_g, gs)
    assert_fp16_close(host(y), r["y"], r["t"], K // gs, what=f"linear pg M={M}")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M", [1, 3, 130])
def test_linear_w4a8_end_to_end(torch_gpu, oracle, M, gs):
    import w4a8_int8_gemm_amd as w
    N, K = 200, 1024
    x = synth.activations(M, K, seed=M + 2 * gs, outliers=True)
    wt = synth.weights(N, K, seed=9)
    w4_g, s4_g = w.pack_weight_int4(dev(wt), gs)
    w4, s4 = oracle.pack_weight_int4(wt, gs)
    assert_equal(host(w4_g), w4, "packed weights")
    assert_equal(host(s4_g), s4, "int4 scales")
    r = oracle.linear("w4a8", x, w4, s4, gs)
    y = w.linear(w.Mode.W4A8, dev(x), w4_g, s4_g, gs)
    assert_fp16_close(host(y), r["y"], r["t"], K // gs, what=f"linear w4a8 M={M}")


def test_linear_workspace_checks(torch_gpu):
    """A workspace below linear_workspace_size() is refused by the binding and,
    called through the C ABI directly, by the library (W4A8_ERR_WORKSPACE,
    nothing launched)."""
    import ctypes
    import torch
    import w4a8_int8_gemm_amd as w
    x = dev(synth.activations(8, 256))
    wq = torch.zeros((16, 256), dtype=torch.int8, device="cuda")
    sw = torch.ones((16,), dtype=torch.float32, device="cuda")
    y = torch.empty((8, 16), dtype=torch.float16, device="cuda")
    small = torch.empty((64,), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        w.linear(w.Mode.W8A8_PC, x, wq, sw, workspace=small)
    P = ctypes.c_void_p
    st = w.lib().linear(int(w.Mode.W8A8_PC), P(x.data_ptr()), 8, 256, P(wq.data_ptr()),
                        P(sw.data_ptr()), 0, 16, P(y.data_ptr()), P(small.data_ptr()), 64,
                        P(torch.cuda.current_stream().cuda_stream))
    assert st == w.Status.ERR_WORKSPACE, st


def test_int8_mv_rounds_to_nearest_even(torch_gpu, oracle):
    """amax = 127 gives s = 1 exactly and integer x gives codes = x; with unit
    weight scales y[n] = fp16(c[n]) is fixed bit for bit (many ties)."""
    import w4a8_int8_gemm_amd as w
    K, N = 2560, 4096
    rng = np.random.default_rng(5)
    x = rng.integers(-127, 128, size=K).astype(np.float16)
    x[7] = 127
    wq = synth.int8_codes(N, K, 21)
    sw = np.ones(N, np.float32)
    r = oracle.int8_mv(x, wq, sw)
    assert r["sa"][0] == 1.0
    y = host(w.int8_mv(dev(x), dev(wq), dev(sw)))
    assert_equal(y.view(np.uint16), r["y"][0].view(np.uint16), "fp16 bits")
