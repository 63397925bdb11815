"""GPU parity: activation and weight quantization, bit for bit against the oracle."""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


QUANT_SHAPES = [
    (16, 256), (1, 2560), (37, 2560), (128, 2560), (3, 14336), (5, 16), (7, 8), (9, 520),
    (2, 16384), (3, 16000),        # the largest register-resident rows (full, ragged)
    (4, 12288), (3, 12000),
    (3, 20480), (2, 16392),        # the two-pass kernel beyond them
    (130, 4096),
]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_quantize_act_per_token(torch_gpu, oracle, M, K):
    import w4a8_int8_gemm_amd as w
    print(f"quantize_act per-token M={M} K={K}", flush=True)
    x = synth.activations(M, K, seed=M + K, outliers=True)
    x[M // 2] = 0                                  # an all-zero token
    xq, xs = w.quantize_act(dev(x))
    want_q, want_s = oracle.quantize_act(x)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,K", [(16, 256), (33, 4096), (5, 14336), (2, 128)])
def test_quantize_act_per_group(torch_gpu, oracle, M, K, gs):
    import w4a8_int8_gemm_amd as w
    if K % gs:
        pytest.skip("K not a multiple of gs")
    print(f"quantize_act per-group M={M} K={K} gs={gs}", flush=True)
    x = synth.activations(M, K, seed=3, outliers=True)
    x[0, :gs] = 0                                  # an all-zero group
    xq, xs = w.quantize_act(dev(x), gs)
    want_q, want_s = oracle.quantize_act(x, gs)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


def test_quantize_act_full_headline(torch_gpu, oracle):
    """The headline activation at full size (4096 x 2560, outlier channels/tokens)."""
    import w4a8_int8_gemm_amd as w
    x = synth.activations(4096, 2560, seed=0, outliers=True)
    xq, xs = w.quantize_act(dev(x))
    want_q, want_s = oracle.quantize_act(x)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


def test_quantize_near_half_inputs(torch_gpu, oracle):
    """Rows built so that many x/s land within a few ulp of a half-integer:
    the inputs where the kernels' guarded fast path must defer to division."""
    import w4a8_int8_gemm_amd as w
    rng = np.random.default_rng(9)
    rows = []
    for _ in range(64):
        amax = np.float16(rng.uniform(0.01, 3000.0))
        s = np.float32(amax) / np.float32(127)
        k = rng.integers(0, 127, size=255).astype(np.float32)
        cand = (s * (k + np.float32(0.5))).astype(np.float16)
        cand = np.minimum(np.abs(cand), amax) * np.where(rng.random(255) < 0.5, -1, 1).astype(np.float16)
        rows.append(np.concatenate([[amax], cand]).astype(np.float16))
    x = np.stack(rows)
    xq, xs = w.quantize_act(dev(x))
    want_q, want_s = oracle.quantize_act(x)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


def _near_half_slices(rng, n, width, frac):
    """n slices of `width` fp16 values: the slice's amax first, then values
    s (k + 1/2) (s = amax / 127) with probability `frac`, Gaussian values
    below amax otherwise -- so that some chunks of a slice need the division
    rule and others do not."""
    out = []
    for _ in range(n):
        amax = np.float16(rng.uniform(0.01, 3000.0))
        s = np.float32(amax) / np.float32(127)
        k = rng.integers(0, 127, size=width - 1).astype(np.float32)
        half = (s * (k + np.float32(0.5))).astype(np.float16)
        plain = (rng.standard_normal(width - 1) * np.float32(amax) / 4).astype(np.float16)
        v = np.where(rng.random(width - 1) < frac, half, plain)
        v = np.minimum(np.abs(v), amax) * np.where(rng.random(width - 1) < 0.5, -1, 1).astype(np.float16)
        out.append(np.concatenate([[amax], v]).astype(np.float16))
    return np.stack(out)


@pytest.mark.parametrize("M,K", [(64, 2560), (16, 4096), (8, 20480)])
def test_quantize_near_half_wide_rows(torch_gpu, oracle, M, K):
    """Whole rows (register-resident and two-pass kernels) where a few chunks
    per row need the division rule and the rest take the fast rule."""
    import w4a8_int8_gemm_amd as w
    print(f"quantize_act near-half per-token M={M} K={K}", flush=True)
    rng = np.random.default_rng(K + M)
    x = _near_half_slices(rng, M, K, 0.004)
    x[M // 2] = 0                                  # an all-zero token
    xq, xs = w.quantize_act(dev(x))
    want_q, want_s = oracle.quantize_act(x)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,K", [(8, 2048), (12, 4096), (6, 14336)])
def test_quantize_near_half_per_group(torch_gpu, oracle, M, K, gs):
    """Per-group slices (one-shot rows up to K = 4096, batched beyond) with
    near-half values in some groups, an all-zero group, and plain groups."""
    import w4a8_int8_gemm_amd as w
    print(f"quantize_act near-half per-group M={M} K={K} gs={gs}", flush=True)
    rng = np.random.default_rng(K + gs)
    x = _near_half_slices(rng, M * K // gs, gs, 0.05).reshape(M, K)
    x[1, gs:2 * gs] = 0                            # an all-zero group
    xq, xs = w.quantize_act(dev(x), gs)
    want_q, want_s = oracle.quantize_act(x, gs)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


def _exact_tie_slices(rng, n, width, qmax):
    """n slices whose amax is qmax 2^k, so that s = 2^k exactly, holding
    values (j + 1/2) 2^k: x / s is then exactly a half-integer (rounded away
    from zero by the rule); the rest of each slice is Gaussian below amax."""
    out = []
    for _ in range(n):
        k = int(rng.integers(-10, 6))
        amax = np.float16(qmax * 2.0 ** k)
        j = rng.integers(0, qmax, size=width - 1)
        tie = ((j + 0.5) * 2.0 ** k).astype(np.float16)
        plain = np.clip(rng.standard_normal(width - 1) * float(amax) / 3, -float(amax), float(amax))
        v = np.where(rng.random(width - 1) < 0.3, tie, plain.astype(np.float16))
        v = v * np.where(rng.random(width - 1) < 0.5, -1, 1)
        out.append(np.concatenate([[amax], v]).astype(np.float16))
    return np.stack(out)


@pytest.mark.parametrize("M,K", [(32, 2560), (8, 4096), (4, 20480)])
def test_quantize_exact_ties_per_token(torch_gpu, oracle, M, K):
    import w4a8_int8_gemm_amd as w
    print(f"quantize_act exact ties per-token M={M} K={K}", flush=True)
    x = _exact_tie_slices(np.random.default_rng(K), M, K, 127)
    xq, xs = w.quantize_act(dev(x))
    want_q, want_s = oracle.quantize_act(x)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


@pytest.mark.parametrize("gs", [64, 128])
def test_quantize_exact_ties_per_group(torch_gpu, oracle, gs):
    import w4a8_int8_gemm_amd as w
    M, K = 8, 4096
    print(f"quantize_act exact ties per-group M={M} K={K} gs={gs}", flush=True)
    x = _exact_tie_slices(np.random.default_rng(gs), M * K // gs, gs, 127).reshape(M, K)
    xq, xs = w.quantize_act(dev(x), gs)
    want_q, want_s = oracle.quantize_act(x, gs)
    assert_equal(host(xs), want_s, "scales")
    assert_equal(host(xq), want_q, "codes")


@pytest.mark.parametrize("gs", [64, 128])
def test_pack_weight_int4_exact_ties(torch_gpu, oracle, gs):
    """int4 weights (qmax 7) with exact half-integer quotients in every group."""
    import w4a8_int8_gemm_amd as w
    N, K = 24, 1024
    print(f"pack_weight_int4 exact ties N={N} K={K} gs={gs}", flush=True)
    wt = _exact_tie_slices(np.random.default_rng(gs + 1), N * K // gs, gs, 7).reshape(N, K)
    wq, sw = w.pack_weight_int4(dev(wt), gs)
    want_q, want_s = oracle.pack_weight_int4(wt, gs)
    assert_equal(host(sw), want_s, "scales")
    assert_equal(host(wq), want_q, "packed codes")


@pytest.mark.parametrize("gs", [0, 64, 128])
def test_quantize_weight_int8(torch_gpu, oracle, gs):
    import w4a8_int8_gemm_amd as w
    wt = synth.weights(300, 2560, seed=1)
    wq, sw = w.quantize_weight_int8(dev(wt), gs)
    want_q, want_s = oracle.quantize_weight_int8(wt, gs)
    assert_equal(host(sw), want_s, "scales")
    assert_equal(host(wq), want_q, "codes")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", [(300, 2560), (17, 128), (64, 4096)])
def test_pack_weight_int4(torch_gpu, oracle, N, K, gs):
    import w4a8_int8_gemm_amd as w
    if K % gs:
        pytest.skip("K not a multiple of gs")
    wt = synth.weights(N, K, seed=2)
    w4, sw = w.pack_weight_int4(dev(wt), gs)
    want_w4, want_s = oracle.pack_weight_int4(wt, gs)
    assert_equal(host(sw), want_s, "scales")
    assert_equal(host(w4), want_w4, "packed codes")


def test_empty_quantize(torch_gpu):
    import torch
    import w4a8_int8_gemm_amd as w
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    xq, xs = w.quantize_act(x)
    assert xq.shape == (0, 256) and xs.shape == (0,)


def test_bad_arguments_raise_on_gpu(torch_gpu):
    import torch
    import w4a8_int8_gemm_amd as w
    x = torch.zeros((4, 12), dtype=torch.float16, device="cuda")
    with pytest.raises(w.W4A8Error) as e:
        w.quantize_act(x)
    assert e.value.status == w.Status.ERR_SHAPE
    x = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(w.W4A8Error):
        w.quantize_act(x, 96)
