"""linear_noalloc(): linear() without a workspace (the activation codes in the
library's static device array), for callers that cannot allocate.

Called through the C ABI and compared byte for byte with linear() on the
same inputs (same kernels, so the same bytes), on two calls in a row with the
second one smaller -- the array keeps the first call's contents, which the
second must not depend on -- for every mode; a size beyond the array is
refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, dev, host, require_gpu

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


def _call_noalloc(w, mode, x, wt, sw, gs, y):
    import torch
    P = ctypes.c_void_p
    M, K = x.shape
    return w.lib().linear_noalloc(int(mode), P(x.data_ptr()), M, K, P(wt.data_ptr()),
                                  P(sw.data_ptr()), gs, wt.shape[0], P(y.data_ptr()),
                                  P(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("mode,gs", [("pc", 0), ("pg", 128), ("pg", 64), ("w4a8", 128)])
def test_noalloc_matches_linear(torch_gpu, mode, gs):
    import torch
    import w4a8_int8_gemm_amd as w
    Mode = {"pc": w.Mode.W8A8_PC, "pg": w.Mode.W8A8_PG, "w4a8": w.Mode.W4A8}[mode]
    N, K = 1536, 2048
    wt = dev(synth.weights(N, K, seed=11))
    if mode == "w4a8":
        wq, sw = w.pack_weight_int4(wt, gs)
    else:
        wq, sw = w.quantize_weight_int8(wt, gs)
    # two calls in a row, the second smaller (the array keeps the first's data)
    for M, seed in ((1000, 1), (300, 2)):
        print(f"linear_noalloc mode={mode} gs={gs} M={M}", flush=True)
        x = dev(synth.activations(M, K, seed=seed, outliers=True))
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        assert w.linear_workspace_size(Mode, M, K, gs) <= SCRATCH_BYTES
        st = _call_noalloc(w, Mode, x, wq, sw, gs, y)
        assert st == 0, w.lib().w4a8_last_error().decode()
        y_ref = w.linear(Mode, x, wq, sw, gs)
        assert_equal(host(y).view(np.uint16), host(y_ref).view(np.uint16),
                     f"linear_noalloc vs linear, M={M}")


def test_noalloc_wrapper_and_decode(torch_gpu):
    """The torch wrapper, and M = 1 (the matrix-vector path, no scratch)."""
    import w4a8_int8_gemm_amd as w
    N, K = 512, 1024
    wq, sw = w.quantize_weight_int8(dev(synth.weights(N, K, seed=3)))
    for M in (64, 1):
        x = dev(synth.activations(M, K, seed=M))
        a = host(w.linear_noalloc(w.Mode.W8A8_PC, x, wq, sw))
        b = host(w.linear(w.Mode.W8A8_PC, x, wq, sw))
        assert_equal(a.view(np.uint16), b.view(np.uint16), f"wrapper M={M}")


def test_noalloc_refuses_beyond_the_array(torch_gpu):
    """M * K codes beyond 64 MiB: W4A8_ERR_WORKSPACE, nothing launched (the
    tensors passed are small; the size check comes before any use of them)."""
    import torch
    import w4a8_int8_gemm_amd as w
    K, N = 4096, 64
    M = SCRATCH_BYTES // K + 1
    assert w.linear_workspace_size(w.Mode.W8A8_PC, M, K, 0) > SCRATCH_BYTES
    x = torch.empty((16, K), dtype=torch.float16, device="cuda")
    wq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sw = torch.ones((N,), dtype=torch.float32, device="cuda")
    y = torch.empty((16, N), dtype=torch.float16, device="cuda")
    P = ctypes.c_void_p
    st = w.lib().linear_noalloc(int(w.Mode.W8A8_PC), P(x.data_ptr()), M, K, P(wq.data_ptr()),
                                P(sw.data_ptr()), 0, N, P(y.data_ptr()),
                                P(torch.cuda.current_stream().cuda_stream))
    assert st == w.Status.ERR_WORKSPACE, st
    assert "static array" in w.lib().w4a8_last_error().decode()
    torch.cuda.synchronize()
