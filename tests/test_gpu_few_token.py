"""Bit-exact checks of the few-token and decode kernels.

The few-token products (1-4 tokens, behind w8a8_gemm_pc and w4a8_gemm) and
the decode matrix-vector kernels never export their int32 sums, so their
arithmetic is pinned two other ways:

* With power-of-two scales every rescale is exact in fp32 (the int32 sums
  convert exactly and a power of two only moves the exponent), so the fp16
  output is fp16(the exact value) on both sides: the GPU result must equal the
  oracle's bit for bit.  Any wrong code, partial sum or fold shows.
* With arbitrary scales the per-channel few-token product and int8_mv promise
  the tiled GEMM's own bits (same int32 sums, same fp32 operation order).  The
  tiled GEMM runs when the same rows are padded to five tokens (rows are
  independent), and the configuration query confirms which kernel each call
  runs.
* The per-group decode kernel quantizes the token itself: a token whose
  groups have absmax 127 * 2^j has scales 2^j exactly, and values placed on
  half-integer multiples exercise the rounding rule (ties away from zero).
"""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def pow2(shape, seed, lo, hi):
    """Powers of two 2^e, e drawn from [lo, hi]."""
    rng = np.random.default_rng([seed, 99])
    return np.ldexp(np.ones(shape, np.float32), rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


FEW_PC = [(1, 10240, 2560), (2, 10240, 2560), (3, 10240, 2560), (4, 10240, 2560),
          (1, 333, 2048), (4, 333, 2048), (2, 4099, 4096), (4, 777, 16384), (3, 129, 64)]


@pytest.mark.parametrize("M,N,K", FEW_PC)
def test_few_token_pc_exact(torch_gpu, oracle, M, N, K):
    import w4a8_int8_gemm_amd as w
    print(f"few-token pc M={M} N={N} K={K}", flush=True)
    assert w.gemm_tile_config(w.GemmOp.GEMM_PC, M, N, K)["bm"] == 0   # the few-token form
    xq, wq = synth.int8_codes(M, K, M + K, 0), synth.int8_codes(N, K, N + K, 1)
    sa, sw = pow2(M, M, -6, -4), pow2(N, N, -6, -4)
    y_ref = oracle.epilogue_pc(oracle.gemm_i32(xq, wq), sa, sw)
    y = host(w.w8a8_gemm_pc(dev(xq), dev(sa), dev(wq), dev(sw)))
    assert_equal(bits(y), bits(y_ref), "fp16 bits, power-of-two scales")


@pytest.mark.parametrize("M,N,K", FEW_PC)
def test_few_token_pc_equals_tiled_gemm(torch_gpu, M, N, K):
    import w4a8_int8_gemm_amd as w
    assert w.gemm_tile_config(w.GemmOp.GEMM_PC, 5, N, K)["bm"] > 0    # five tokens: tiled
    xq = synth.int8_codes(5, K, 3 * M + K, 0)
    wq = synth.int8_codes(N, K, N + K, 1)
    sa, sw = synth.scales(5, 0, M, 0, 3.0), synth.scales(N, 0, N, 1)
    y_few = host(w.w8a8_gemm_pc(dev(xq[:M]), dev(sa[:M]), dev(wq), dev(sw)))
    y_tiled = host(w.w8a8_gemm_pc(dev(xq), dev(sa), dev(wq), dev(sw)))[:M]
    assert_equal(bits(y_few), bits(y_tiled), "few-token vs tiled GEMM bytes")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", [(1, 6144, 4096), (2, 1001, 1024), (3, 333, 2048),
                                   (4, 4099, 4096), (4, 100, 256)])
def test_few_token_w4a8_exact(torch_gpu, oracle, M, N, K, gs):
    import w4a8_int8_gemm_amd as w
    print(f"few-token w4a8 M={M} N={N} K={K} gs={gs}", flush=True)
    assert w.gemm_tile_config(w.GemmOp.GEMM_W4A8, M, N, K, gs)["bm"] == 0
    G = K // gs
    xq, w4 = synth.int8_codes(M, K, M + K, 0), synth.packed_int4(N, K, N + K, 1)
    sa, sw = pow2(M, M, -6, -4), pow2((N, G), N + gs, -5, -4)
    p = oracle.gemm_partials(xq, oracle.unpack_int4(w4, K), gs)
    y_ref, _ = oracle.epilogue_w4a8(p, sa, sw)
    y = host(w.w4a8_gemm(dev(xq), dev(sa), dev(w4), dev(sw), gs))
    assert_equal(bits(y), bits(y_ref), "fp16 bits, power-of-two scales")


@pytest.mark.parametrize("N,K", [(10240, 2560), (333, 4096), (64, 14336), (100, 64)])
def test_int8_mv_equals_tiled_gemm(torch_gpu, oracle, N, K):
    """The decode kernel's bytes are the tiled GEMM's at M = 1 (the token's
    codes and scale, exported, are the quantizer's)."""
    import w4a8_int8_gemm_amd as w
    x = synth.activations(5, K, seed=K + 1, outliers=True)
    wq, sw = oracle.quantize_weight_int8(synth.weights(N, K, seed=N))
    y_mv, xq1, xs1 = w.int8_mv(dev(x[0]), dev(wq), dev(sw), return_codes=True)
    xq, xs = w.quantize_act(dev(x))
    assert_equal(host(xq1), host(xq)[0], "token codes")
    assert_equal(host(xs1), host(xs)[:1], "token scale")
    y_tiled = host(w.w8a8_gemm_pc(xq, xs, dev(wq), dev(sw)))[0]
    assert_equal(bits(host(y_mv)), bits(y_tiled), "int8_mv vs tiled GEMM bytes")


def _token_pow2_groups(K, gs, seed):
    """fp16 token whose group g has absmax exactly 127 * 2^j_g (so its scale is
    2^j_g): integer and half-integer multiples of 2^j_g, ties included."""
    rng = np.random.default_rng([seed, 7])
    G = K // gs
    j = rng.integers(-6, -4, size=G)
    half_steps = rng.integers(-254, 255, size=K).astype(np.float64)      # multiples of 1/2
    x = np.empty(K, np.float64)
    for g in range(G):
        sl = slice(g * gs, (g + 1) * gs)
        x[sl] = half_steps[sl] * 0.5 * 2.0 ** j[g]
        x[g * gs + rng.integers(0, gs)] = 127.0 * 2.0 ** j[g] * (1 if g % 2 else -1)
    xh = x.astype(np.float16)
    assert np.array_equal(xh.astype(np.float64), x)                      # exactly representable
    return xh


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", [(300, 1024), (4096, 2048), (77, 4096)])
def test_w8a8_mv_pg_exact(torch_gpu, oracle, N, K, gs):
    import w4a8_int8_gemm_amd as w
    print(f"w8a8_mv_pg exact N={N} K={K} gs={gs}", flush=True)
    G = K // gs
    x = _token_pow2_groups(K, gs, K + gs)
    xo, so = oracle.quantize_act(x.reshape(1, K), gs)
    assert np.all(np.log2(so) == np.round(np.log2(so)))                  # scales are powers of two
    assert np.any(np.abs(x.astype(np.float64) / np.repeat(so[0], gs)) % 1 == 0.5)  # ties present
    wq = synth.int8_codes(N, K, N, 3)
    sw = pow2((N, G), N + K, -7, -6)
    y_ref, _ = oracle.epilogue_pg(oracle.gemm_partials(xo, wq, gs), so, sw)
    y = host(w.w8a8_mv_pg(dev(x), dev(wq), dev(sw), gs))
    assert_equal(bits(y), bits(y_ref[0]), "fp16 bits (codes, group scales and fold exact)")


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("N,K", [(300, 1024), (6144, 4096), (77, 2048)])
def test_w4a8_mv_exact(torch_gpu, oracle, N, K, gs):
    import w4a8_int8_gemm_amd as w
    print(f"w4a8_mv exact N={N} K={K} gs={gs}", flush=True)
    G = K // gs
    x = _token_pow2_groups(K, K, K + 3 * gs)                             # one slice: per token
    xo, so = oracle.quantize_act(x.reshape(1, K), 0)
    assert np.log2(so[0]) == np.round(np.log2(so[0]))
    w4 = synth.packed_int4(N, K, N, 4)
    sw = pow2((N, G), N + 2 * K, -5, -4)
    y_ref, _ = oracle.epilogue_w4a8(oracle.gemm_partials(xo, oracle.unpack_int4(w4, K), gs), so, sw)
    y = host(w.w4a8_mv(dev(x), dev(w4), dev(sw), gs))
    assert_equal(bits(y), bits(y_ref[0]), "fp16 bits (codes, scales and fold exact)")
