"""Pins of the oracle's weight-only int8 product (the pages' W8A16 baseline,
"cider" post, section on its performance results): against exact rational
arithmetic on small inputs, and closed forms.  CPU only."""
from fractions import Fraction

import numpy as np

import synth
from tests.exact import f16_bits_to_fraction, f32_bits_to_fraction, to_f16


def _exact(x, wq, sw):
    M, K = x.shape
    N = wq.shape[0]
    xb = x.view(np.uint16)
    sb = sw.view(np.uint32)
    y = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        xf = [f16_bits_to_fraction(int(b)) for b in xb[m]]
        for n in range(N):
            s = sum(xf[k] * int(wq[n, k]) for k in range(K)) * f32_bits_to_fraction(int(sb[n]))
            y[m, n] = float(to_f16(s))
    return y


def test_w8a16_matches_exact_rounding(oracle):
    x = synth.activations(6, 96, seed=3)
    wt = synth.weights(9, 96, seed=4)
    wq, sw = oracle.quantize_weight_int8(wt, 0)
    y, t = oracle.w8a16(x, wq, sw)
    assert np.array_equal(y.astype(np.float64), _exact(x, wq, sw))
    # T is the scaled sum of |products|
    ref_t = np.abs(x.astype(np.float64))[:, None, :] * np.abs(wq.astype(np.float64))[None, :, :]
    assert np.allclose(t, ref_t.sum(-1) * sw.astype(np.float64)[None, :], rtol=1e-12)


def test_w8a16_closed_forms(oracle):
    # one-hot activation row: y[n] = fp16(x * wq[n, k] * sw[n]); constant weight row: x row sum
    K = 128
    x = np.zeros((2, K), dtype=np.float16)
    x[0, 17] = np.float16(0.375)
    x[1, :] = np.float16(0.5)
    wq = np.zeros((3, K), dtype=np.int8)
    wq[0, 17] = -96
    wq[1, :] = 3
    wq[2, :] = np.arange(K) % 255 - 127
    sw = np.array([0.25, 2.0 ** -3, 1.0], dtype=np.float32)
    y, _ = oracle.w8a16(x, wq, sw)
    assert y[0, 0] == np.float16(0.375 * -96 * 0.25)
    assert y[0, 1] == np.float16(0.375 * 3 * 2.0 ** -3)
    assert y[1, 1] == np.float16(0.5 * 3 * K * 2.0 ** -3)
    assert y[1, 2] == np.float16(0.5 * float((np.arange(K) % 255 - 127).sum()))
    assert y[0, 2] == np.float16(0.375 * (17 - 127))


def _exact_w4a16(x, codes, sw, gs):
    """fp16(fl32(code * s)) per weight, then the exact sum rounded to fp16."""
    from tests.exact import to_f32
    M, K = x.shape
    N = codes.shape[0]
    xb = x.view(np.uint16)
    sb = sw.view(np.uint32)
    wd = [[to_f16(to_f32(int(codes[n, k]) * f32_bits_to_fraction(int(sb[n, k // gs]))))
           for k in range(K)] for n in range(N)]
    y = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        xf = [f16_bits_to_fraction(int(b)) for b in xb[m]]
        for n in range(N):
            y[m, n] = float(to_f16(sum(xf[k] * wd[n][k] for k in range(K))))
    return y


def test_w4a16_matches_exact_rounding(oracle):
    x = synth.activations(5, 128, seed=5)
    w4, s4 = oracle.pack_weight_int4(synth.weights(7, 128, seed=6), 64)
    y, t = oracle.w4a16(x, w4, s4, 64)
    codes = oracle.unpack_int4(w4, 128)
    assert np.array_equal(y.astype(np.float64), _exact_w4a16(x, codes, s4, 64))
    assert np.all(t >= np.abs(y.astype(np.float64)) * (1 - 2.0 ** -10))


def test_w4a16_every_code_and_rounding(oracle):
    # one-hot activations read single dequantized weights: every code -8..7,
    # and a scale whose products with odd codes need rounding to fp16
    K = 64
    codes = np.zeros((16, K), dtype=np.int8)
    codes[:, 3] = np.arange(-8, 8)
    w4 = oracle.pack_int4(codes)
    s = np.float32(0.1)                      # not a power of two: products round
    sw = np.full((16, 1), s, dtype=np.float32)
    x = np.zeros((1, K), dtype=np.float16)
    x[0, 3] = np.float16(1.0)
    y, _ = oracle.w4a16(x, w4, sw, 64)
    want = np.array([np.float16(np.float32(c) * s) for c in range(-8, 8)], dtype=np.float16)
    assert np.array_equal(y[0], want)
