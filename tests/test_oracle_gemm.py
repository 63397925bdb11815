"""Pins for the oracle's int8 GEMMs and rescale epilogues (CPU only).

Independent references: pure-Python integer loops, numpy float64 matmul
(exact while |C| < 2^53), exact rational arithmetic for the fp16 rounding,
hand-worked values, closed forms, cross-mode identities, and the error bound
that ties the quantized result to an fp64 GEMM of the fp16 sources.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import yaml

import synth
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.yaml")


@pytest.fixture(scope="module")
def gold():
    with open(GOLDEN) as f:
        return yaml.safe_load(f)


def _py_gemm(a, b):
    return [[sum(int(a[m][k]) * int(b[n][k]) for k in range(len(a[m]))) for n in range(len(b))]
            for m in range(len(a))]


# ----------------------------------------------------------------------------- golden

def test_golden_pc(oracle, gold):
    g = gold["gemm_pc"]
    c = oracle.gemm_i32(np.array(g["xq"], np.int8), np.array(g["wq"], np.int8))
    assert c.tolist() == g["C"]
    y = oracle.epilogue_pc(c, np.array(g["sa"], np.float32), np.array(g["sw"], np.float32))
    assert y.astype(np.float64).tolist() == g["y"]


def test_golden_pg(oracle, gold):
    g = gold["gemm_pg"]
    p = oracle.gemm_partials(np.array(g["xq"], np.int8), np.array(g["wq"], np.int8), g["gs"])
    assert p.tolist() == g["P"]
    y, _ = oracle.epilogue_pg(p, np.array(g["sa"], np.float32), np.array(g["sw"], np.float32))
    assert y.astype(np.float64).tolist() == g["y"]


def test_golden_w4a8(oracle, gold):
    g = gold["w4a8"]
    xq = np.array(g["xq"], np.int8)
    codes = oracle.unpack_int4(np.array(g["packed"], np.uint8), xq.shape[1])
    p = oracle.gemm_partials(xq, codes, g["gs"])
    assert p.tolist() == g["P"]
    y, _ = oracle.epilogue_w4a8(p, np.array(g["sa"], np.float32), np.array(g["sw"], np.float32))
    assert y.astype(np.float64).tolist() == g["y"]


# ----------------------------------------------------------------------------- integer sums

def test_gemm_vs_python_bigint(oracle):
    rng = np.random.default_rng(0)
    for M, N, K in [(1, 1, 1), (3, 5, 7), (6, 4, 64), (2, 8, 256)]:
        a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        a[0, : min(K, 4)] = 127
        b[0, : min(K, 4)] = -127
        assert oracle.gemm_i32(a, b).tolist() == _py_gemm(a.tolist(), b.tolist())
        gs = K if K < 4 else K // 4
        if K % gs == 0:
            p = oracle.gemm_partials(a, b, gs)
            for g in range(K // gs):
                sl = slice(g * gs, (g + 1) * gs)
                assert p[g].tolist() == _py_gemm(a[:, sl].tolist(), b[:, sl].tolist())


def test_gemm_vs_float64_matmul(oracle):
    # integer-valued float64 matmul is exact while |C| < 2^53
    x = synth.activations(96, 1024, seed=0, outliers=True)
    w = synth.weights(160, 1024, seed=0)
    xq, _ = oracle.quantize_act(x)
    wq, _ = oracle.quantize_weight_int8(w)
    c = oracle.gemm_i32(xq, wq)
    ref = xq.astype(np.float64) @ wq.astype(np.float64).T
    np.testing.assert_array_equal(c.astype(np.float64), ref)


def test_partials_identities(oracle):
    rng = np.random.default_rng(1)
    a = rng.integers(-127, 128, size=(24, 512)).astype(np.int8)
    b = rng.integers(-127, 128, size=(40, 512)).astype(np.int8)
    c = oracle.gemm_i32(a, b)
    for gs in (64, 128):
        p = oracle.gemm_partials(a, b, gs)
        np.testing.assert_array_equal(p.astype(np.int64).sum(axis=0), c)
    np.testing.assert_array_equal(oracle.gemm_partials(a, b, 512)[0], c)


def test_gemm_closed_forms(oracle):
    # one-hot activation row v*e_k quantizes to +-127*e_k, so C[m,:] = +-127*Wq[:,k]
    K = 256
    x = np.zeros((3, K), np.float16)
    x[0, 5] = 3.0
    x[1, 200] = -0.125
    x[2, 0] = 1e-3
    w = synth.weights(64, K, seed=9)
    wq, _ = oracle.quantize_weight_int8(w)
    xq, _ = oracle.quantize_act(x)
    c = oracle.gemm_i32(xq, wq)
    np.testing.assert_array_equal(c[0], 127 * wq[:, 5].astype(np.int32))
    np.testing.assert_array_equal(c[1], -127 * wq[:, 200].astype(np.int32))
    np.testing.assert_array_equal(c[2], 127 * wq[:, 0].astype(np.int32))
    # a constant weight row q_w gives C[m, n] = q_w * sum_k Xq[m, k]
    wc = np.full((2, K), 0.5, np.float16)
    wc[1] = -0.5
    wcq, _ = oracle.quantize_weight_int8(wc)
    xr = synth.activations(5, K, seed=2)
    xrq, _ = oracle.quantize_act(xr)
    c = oracle.gemm_i32(xrq, wcq)
    rs = xrq.astype(np.int32).sum(axis=1)
    np.testing.assert_array_equal(c[:, 0], 127 * rs)
    np.testing.assert_array_equal(c[:, 1], -127 * rs)


def test_gemm_int32_overflow_detected(oracle):
    K = 140000                                 # 127^2 * K > 2^31 - 1
    a = np.full((1, K), 127, np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_i32(a, a)
    K = 133144                                 # largest K with 127^2 * K < 2^31
    a = np.full((1, K), 127, np.int8)
    assert int(oracle.gemm_i32(a, a)[0, 0]) == 127 * 127 * K


# ----------------------------------------------------------------------------- epilogues

def _exact_f16(r: Fraction) -> float:
    return float(exact.to_f16(r))


def test_epilogue_pc_vs_exact(oracle):
    rng = np.random.default_rng(2)
    M, N = 20, 30
    c = rng.integers(-40_000_000, 40_000_000, size=(M, N)).astype(np.int32)
    c[0, :5] = [0, 1, -1, 2**28, -(2**28)]
    sa = (rng.random(M) * 0.05).astype(np.float32)
    sw = (rng.random(N) * 2e-4 + 1e-6).astype(np.float32)
    y = oracle.epilogue_pc(c, sa, sw)
    for m in range(M):
        for n in range(N):
            want = _exact_f16(Fraction(int(c[m, n])) * Fraction(float(sa[m])) * Fraction(float(sw[n])))
            assert float(y[m, n]) == want, (m, n)


def test_epilogue_pg_and_w4a8_vs_exact(oracle):
    rng = np.random.default_rng(3)
    G, M, N = 6, 5, 7
    p = rng.integers(-1_000_000, 1_000_000, size=(G, M, N)).astype(np.int32)
    sa = (rng.random((M, G)) * 0.05).astype(np.float32)
    sw = (rng.random((N, G)) * 2e-4).astype(np.float32)
    y, t = oracle.epilogue_pg(p, sa, sw)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(int(p[g, m, n])) * Fraction(float(sa[m, g])) * Fraction(float(sw[n, g]))
                     for g in range(G)]
            assert float(y[m, n]) == _exact_f16(sum(terms))
            assert abs(Fraction(float(t[m, n])) - sum(abs(v) for v in terms)) <= 1e-12 * t[m, n]
    sa1 = sa[:, 0].copy()
    y4, _ = oracle.epilogue_w4a8(p, sa1, sw)
    for m in range(M):
        for n in range(N):
            tot = sum(Fraction(int(p[g, m, n])) * Fraction(float(sw[n, g])) for g in range(G))
            assert float(y4[m, n]) == _exact_f16(Fraction(float(sa1[m])) * tot)


# ----------------------------------------------------------------------------- accuracy bound

def _ulp16(y):
    a = np.abs(y.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0**-14)))
    return 2.0 ** (e - 10)


def test_pc_error_bound_vs_fp64_gemm(oracle):
    """|Y - x.w| <= (1/2 + 2^-17)(sa*sum|w| + sw*sum|x_hat|) + ulp16(Y)/2, elementwise,
    where x.w is the fp64 GEMM of the fp16 sources and x_hat = q*sa."""
    M, N, K = 16, 512, 256
    x = synth.activations(M, K, seed=0)
    w = synth.weights(N, K, seed=0)
    wq, sw = oracle.quantize_weight_int8(w)
    r = oracle.w8a8_pc(x, wq, sw)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    xhat = r["xq"].astype(np.float64) * r["sa"][:, None]
    d = 0.5 + 2.0**-17
    bound = d * (r["sa"][:, None] * np.abs(w.astype(np.float64)).sum(1)[None, :]
                 + sw[None, :].astype(np.float64) * np.abs(xhat).sum(1)[:, None])
    bound += 0.5 * _ulp16(r["y"]) + 1e-12
    err = np.abs(r["y"].astype(np.float64) - ref)
    assert np.all(err <= bound)
    # and the bound is not vacuous: the observed error uses a good part of it
    assert (err / bound).max() > 0.05


def test_pg_and_w4a8_error_bound(oracle):
    M, N, K, gs = 8, 64, 512, 128
    x = synth.activations(M, K, seed=4)
    w = synth.weights(N, K, seed=4)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    d = 0.5 + 2.0**-17
    G = K // gs
    wq, sw = oracle.quantize_weight_int8(w, gs)
    r = oracle.w8a8_pg(x, wq, sw, gs)
    xhat = (r["xq"].astype(np.float64).reshape(M, G, gs) * r["sa"][:, :, None])
    wa = np.abs(w.astype(np.float64)).reshape(N, G, gs).sum(2)
    bound = d * (np.einsum("mg,ng->mn", r["sa"].astype(np.float64), wa)
                 + np.einsum("ng,mg->mn", sw.astype(np.float64), np.abs(xhat).sum(2)))
    bound += 0.5 * _ulp16(r["y"]) + 1e-12
    assert np.all(np.abs(r["y"].astype(np.float64) - ref) <= bound)
    # W4A8: int4 weights, codes +-7
    w4, s4 = oracle.pack_weight_int4(w, gs)
    r4 = oracle.w4a8(x, w4, s4, gs)
    xhat = r4["xq"].astype(np.float64) * r4["sa"][:, None]
    xa = np.abs(xhat).reshape(M, G, gs).sum(2)
    bound = d * (r4["sa"][:, None].astype(np.float64) * np.abs(w.astype(np.float64)).sum(1)[None, :]
                 + np.einsum("ng,mg->mn", s4.astype(np.float64), xa))
    bound += 0.5 * _ulp16(r4["y"]) + 1e-12
    assert np.all(np.abs(r4["y"].astype(np.float64) - ref) <= bound)


# ----------------------------------------------------------------------------- dispatch

def test_linear_dispatch(oracle):
    x = synth.activations(3, 256, seed=5)
    w = synth.weights(32, 256, seed=5)
    wq, sw = oracle.quantize_weight_int8(w)
    full = oracle.linear("pc", x, wq, sw)
    for m in range(3):
        mv = oracle.linear("pc", x[m:m + 1], wq, sw)
        np.testing.assert_array_equal(mv["y"][0], full["y"][m])
        np.testing.assert_array_equal(mv["xq"][0], full["xq"][m])
    wq64, sw64 = oracle.quantize_weight_int8(w, 64)
    pg = oracle.linear("pg", x, wq64, sw64, 64)
    assert pg["y"].shape == (3, 32) and pg["p"].shape == (4, 3, 32)
    # per-group with a single group equals per-channel
    one = oracle.w8a8_pg(x, wq, sw[:, None].copy(), 256)
    np.testing.assert_array_equal(one["xq"], full["xq"])
    np.testing.assert_array_equal(one["p"][0], full["c"])
    np.testing.assert_array_equal(one["y"], full["y"])
