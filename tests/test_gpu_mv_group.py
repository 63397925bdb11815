"""GPU parity of the decode matrix-vector kernels with per-group weight scales
(per-group W8A8 and W4A8) against the oracle's per-group pipeline at M = 1,
each side quantizing the fp16 token itself."""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, assert_fp16_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


# (N, K): 4, 8 and 16 weight chunks in flight per lane, rows of several
# passes, 2, 4, 8 and 16 token chunks per thread, N not a multiple of the 16
# rows per workgroup, the smallest and the largest K; 5000 and 6100 rows take
# the 768-thread int4 workgroups on a 256-CU device
SHAPES = [(300, 1024), (129, 2048), (4096, 4096), (1000, 8192), (4096, 14336), (77, 32768),
          (17, 128), (5000, 4096), (6100, 8192)]


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", SHAPES)
def test_w8a8_mv_pg(torch_gpu, oracle, N, K, gs):
    import w4a8_int8_gemm_amd as w
    print(f"w8a8_mv_pg N={N} K={K} gs={gs}", flush=True)
    x = synth.activations(1, K, seed=K + gs, outliers=True)
    wq, sw = oracle.quantize_weight_int8(synth.weights(N, K, seed=N), gs)
    r = oracle.linear("pg", x, wq, sw, gs)
    y = w.w8a8_mv_pg(dev(x[0]), dev(wq), dev(sw), gs)
    assert_fp16_close(host(y), r["y"][0], r["t"][0], K // gs, what=f"pg mv N={N} K={K}")
    # linear() at M = 1 dispatches here
    y2 = w.linear(w.Mode.W8A8_PG, dev(x), dev(wq), dev(sw), gs)
    assert_equal(host(y2)[0], host(y), "linear dispatch to the per-group MV")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", SHAPES)
def test_w4a8_mv(torch_gpu, oracle, N, K, gs):
    import w4a8_int8_gemm_amd as w
    print(f"w4a8_mv N={N} K={K} gs={gs}", flush=True)
    x = synth.activations(1, K, seed=K + 3 * gs, outliers=True)
    w4, s4 = oracle.pack_weight_int4(synth.weights(N, K, seed=N + 1), gs)
    r = oracle.linear("w4a8", x, w4, s4, gs)
    y = w.w4a8_mv(dev(x[0]), dev(w4), dev(s4), gs)
    assert_fp16_close(host(y), r["y"][0], r["t"][0], K // gs, what=f"w4a8 mv N={N} K={K}")
    y2 = w.linear(w.Mode.W4A8, dev(x), dev(w4), dev(s4), gs)
    assert_equal(host(y2)[0], host(y), "linear dispatch to the W4A8 MV")


def test_mv_group_zero_groups(torch_gpu, oracle):
    """All-zero groups of the token get scale 0 and codes 0 (their partial
    sums vanish); an all-zero token gives y = 0."""
    import w4a8_int8_gemm_amd as w
    N, K, gs = 256, 2048, 128
    x = synth.activations(1, K, seed=3, outliers=True)
    x[0, 128:384] = 0                      # groups 1 and 2
    wq, sw = oracle.quantize_weight_int8(synth.weights(N, K, seed=4), gs)
    r = oracle.linear("pg", x, wq, sw, gs)
    y = w.w8a8_mv_pg(dev(x[0]), dev(wq), dev(sw), gs)
    assert_fp16_close(host(y), r["y"][0], r["t"][0], K // gs, what="pg mv with zero groups")
    z = np.zeros((K,), np.float16)
    assert np.all(host(w.w8a8_mv_pg(dev(z), dev(wq), dev(sw), gs)) == 0)
    w4, s4 = oracle.pack_weight_int4(synth.weights(N, K, seed=5), gs)
    assert np.all(host(w.w4a8_mv(dev(z), dev(w4), dev(s4), gs)) == 0)


def test_w4a8_mv_every_nibble(torch_gpu, oracle):
    """Weights that use every int4 code in both nibble positions, integer
    token values with amax 127 (scale 1) and unit weight scales: the sums are
    exact, so the fp16 outputs match the oracle bit for bit."""
    import w4a8_int8_gemm_amd as w
    N, K, gs = 64, 1024, 128
    rng = np.random.default_rng(11)
    codes = rng.integers(-8, 8, size=(N, K))
    w4 = ((codes[:, 0::2] & 0xF) | ((codes[:, 1::2] & 0xF) << 4)).astype(np.uint8)
    s4 = np.ones((N, K // gs), np.float32)
    x = rng.integers(-127, 128, size=(1, K)).astype(np.float16)
    x[0, 5] = 127
    r = oracle.linear("w4a8", x, w4, s4, gs)
    y = host(w.w4a8_mv(dev(x[0]), dev(w4), dev(s4), gs))
    ref = (codes.astype(np.int64) @ x[0].astype(np.int64)).astype(np.float16)
    assert_equal(r["y"][0].view(np.uint16), ref.view(np.uint16), "oracle, exact sums")
    assert_equal(y.view(np.uint16), ref.view(np.uint16), "fp16 bits")
