"""Pins for the oracle's quantizer and fp16 rounding (CPU only).

Each check ties the oracle to something other than itself: exact rational
arithmetic (tests/exact.py), hand-worked values (tests/golden), closed forms
and invariants of the rule s = fl32(amax/qmax), q = clamp(rha(fl32(x/s))).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import yaml

import synth
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.yaml")


def golden():
    with open(GOLDEN) as f:
        return yaml.safe_load(f)


def _f32_frac(v) -> Fraction:
    return exact.f32_bits_to_fraction(int(np.float32(v).view(np.uint32)))


def _f16_frac(v) -> Fraction:
    return exact.f16_bits_to_fraction(int(np.float16(v).view(np.uint16)))


# ----------------------------------------------------------------------------- exact helpers

def test_exact_helper_known_values():
    # fl32(1/3) has the well-known bit pattern 0x3EAAAAAB; fl32(1/127) is 0x3C010204.
    assert exact.to_f32(Fraction(1, 3)) == exact.f32_bits_to_fraction(0x3EAAAAAB)
    assert exact.to_f32(Fraction(1, 127)) == exact.f32_bits_to_fraction(0x3C010204)
    assert exact.to_f16(Fraction(1, 3)) == exact.f16_bits_to_fraction(0x3555)
    assert exact.round_half_away(Fraction(5, 2)) == 3
    assert exact.round_half_away(Fraction(-5, 2)) == -3
    assert exact.round_half_away(Fraction(2**24 - 1, 2**25)) == 0


# ----------------------------------------------------------------------------- fp16 conversions

def test_f16_decode_exhaustive(oracle):
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    finite = [b for b in bits.tolist() if ((b >> 10) & 0x1F) != 31]
    sample = finite[::7] + [0x0001, 0x03FF, 0x0400, 0x7BFF, 0x8001, 0xFBFF]
    got = oracle.f16_to_f64(np.array(sample, dtype=np.uint16).view(np.float16))
    for b, g in zip(sample, got.tolist()):
        assert Fraction(g) == exact.f16_bits_to_fraction(b)


def test_f64_to_f16_golden(oracle):
    for case in golden()["fp16_rounding"]:
        got = float(oracle.f64_to_f16([case["value"]])[0])
        assert got == case["f16"], case


def test_f64_to_f16_ties_and_random(oracle):
    rng = np.random.default_rng(11)
    # midpoints between neighbouring fp16 values: the hard cases for rounding
    h = rng.integers(0, 0x7BFF, size=3000, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = (lo + hi) / 2.0                       # exact in fp64
    vals = np.concatenate([mids, -mids, rng.standard_normal(2000) * 100.0,
                           rng.standard_normal(500) * 1e-6])
    got = oracle.f64_to_f16(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        want = exact.to_f16(Fraction(v))
        if want in (float("inf"), -float("inf")):
            assert g == want
        else:
            assert Fraction(g) == want, (v, g)


# ----------------------------------------------------------------------------- golden examples

def test_quantize_golden(oracle):
    for case in golden()["quantize"]:
        x = np.array([case["x"]], dtype=np.float16)
        q, s = oracle.quantize(x, 0, case["qmax"])
        assert float(s[0]) == case["scale"], case["name"]
        assert q[0].tolist() == case["codes"], case["name"]


def test_pack_int4_golden(oracle):
    for case in golden()["pack_int4"]:
        codes = np.array([case["codes"]], dtype=np.int8)
        packed = oracle.pack_int4(codes)
        assert packed[0].tolist() == case["bytes"]
        assert oracle.unpack_int4(packed, codes.shape[1]).tolist() == codes.tolist()


# ----------------------------------------------------------------------------- brute force

def _quant_vs_exact(oracle, amax_bits: int, xs_bits: np.ndarray, qmax: int):
    """Oracle codes for the row [amax, xs...] against the exact-rational rule."""
    row = np.concatenate([[amax_bits], xs_bits]).astype(np.uint16).view(np.float16)[None, :]
    q, s = oracle.quantize(row, 0, qmax)
    vals = [exact.f16_bits_to_fraction(int(b)) for b in row.view(np.uint16)[0]]
    s_ref, q_ref = exact.quantize_exact(vals, qmax)
    assert _f32_frac(s[0]) == s_ref
    np.testing.assert_array_equal(q[0], np.array(q_ref, dtype=np.int8))


@pytest.mark.parametrize("amax", [1.0, 3.140625, 0.0078125 * 3, 1000.0])
def test_quantize_exhaustive_fp16(oracle, amax):
    """Every finite fp16 x with |x| <= amax, against exact rational arithmetic."""
    a_bits = int(np.float16(amax).view(np.uint16))
    pos = np.arange(0, a_bits + 1, dtype=np.uint16)
    xs = np.concatenate([pos, pos | 0x8000])
    for chunk in np.array_split(xs, max(1, len(xs) // 4096)):
        _quant_vs_exact(oracle, a_bits, chunk, 127)


def test_quantize_random_amax(oracle):
    rng = np.random.default_rng(5)
    for _ in range(150):
        a_bits = int(rng.integers(0x0400, 0x7BFF))
        xs = rng.integers(0, a_bits + 1, size=64, dtype=np.uint16)
        xs |= (rng.integers(0, 2, size=64, dtype=np.uint16) << 15).astype(np.uint16)
        _quant_vs_exact(oracle, a_bits, xs, 127)
        _quant_vs_exact(oracle, a_bits, xs, 7)


def test_near_half_cases_round_away(oracle):
    """Inputs whose fl32(x/s) lies within 2 ulp of a half-integer -- the cases
    where the rounding rule decides the code.  numpy only *finds* candidates
    (fp16 neighbours of s*(k+1/2)); the expected codes come from exact
    rational arithmetic."""
    rng = np.random.default_rng(3)
    a_bits = rng.integers(0x0400, 0x7BFF, size=600).astype(np.uint16)
    amax = a_bits.view(np.float16).astype(np.float32)
    s = amax / np.float32(127)
    k = np.arange(0, 127, dtype=np.float32)
    cand = (s[:, None] * (k[None, :] + np.float32(0.5))).astype(np.float16).view(np.uint16)
    cases = []
    for d in (-1, 0, 1):
        b = (cand.astype(np.int32) + d).clip(0, 0x7BFF).astype(np.uint16)
        x = b.view(np.float16).astype(np.float32)
        t = x / s[:, None]
        near = (x <= amax[:, None]) & (np.abs(t - np.floor(t) - 0.5) <= 2 * np.spacing(t))
        for i, j in zip(*np.nonzero(near)):
            cases.append((int(a_bits[i]), int(b[i, j])))
    assert len(cases) > 300
    pick = rng.choice(len(cases), size=300, replace=False)
    by_amax = {}
    for idx in pick.tolist():
        a, b = cases[idx]
        by_amax.setdefault(a, []).append(b)
    for a, bs in by_amax.items():
        bs = np.array(bs, dtype=np.uint16)
        _quant_vs_exact(oracle, a, np.concatenate([bs, bs | 0x8000]), 127)


# ----------------------------------------------------------------------------- invariants

def test_quantize_invariants(oracle):
    x = synth.activations(64, 512, seed=1, outliers=True)
    for gs in (0, 64, 128):
        q, s = oracle.quantize_act(x, gs)
        s2 = s.reshape(64, -1)
        glen = 512 if gs == 0 else gs
        qg = q.reshape(64, -1, glen).astype(np.int32)
        xg = x.astype(np.float64).reshape(64, -1, glen)
        assert qg.min() >= -127 and qg.max() <= 127
        nz = np.abs(xg).max(axis=2) > 0
        assert np.all(np.abs(qg).max(axis=2)[nz] == 127)        # every nonzero slice hits +-127
        err = np.abs(xg - qg * s2[:, :, None].astype(np.float64))
        assert np.all(err <= s2[:, :, None] * (0.5 + 2.0**-17))  # dequant error bound
        # odd symmetry and row permutation
        qn, sn = oracle.quantize_act(-x, gs)
        np.testing.assert_array_equal(qn, -q)
        np.testing.assert_array_equal(sn, s)
        perm = np.random.default_rng(0).permutation(64)
        qp, sp = oracle.quantize_act(x[perm], gs)
        np.testing.assert_array_equal(qp, q[perm])
        np.testing.assert_array_equal(sp, s[perm])


def test_quantize_power_of_two_scaling(oracle):
    x = synth.activations(8, 256, seed=2)
    q, s = oracle.quantize_act(x, 0)
    for j in (-3, 1, 4):
        xj = (x.astype(np.float32) * np.float32(2.0**j)).astype(np.float16)
        assert np.all(xj.astype(np.float32) == x.astype(np.float32) * np.float32(2.0**j))
        qj, sj = oracle.quantize_act(xj, 0)
        np.testing.assert_array_equal(qj, q)
        np.testing.assert_array_equal(sj, s * np.float32(2.0**j))


def test_quantize_closed_forms(oracle):
    # constant row c: every code is sign(c)*127 and s = fl32(|c|/127)
    for c in (0.3, -7.25, 1000.0):
        row = np.full((1, 100), c, dtype=np.float16)
        q, s = oracle.quantize_act(row, 0)
        assert np.all(q == (127 if c > 0 else -127))
        assert _f32_frac(s[0]) == exact.to_f32(abs(_f16_frac(c)) / 127)
    # zero rows and zero groups
    x = synth.activations(4, 256, seed=3)
    x[1] = 0
    x[2, 64:128] = 0
    q, s = oracle.quantize_act(x, 64)
    assert np.all(s[1] == 0) and np.all(q[1] == 0)
    assert s[2, 1] == 0 and np.all(q[2, 64:128] == 0) and np.all(s[2, [0, 2, 3]] > 0)


def test_quantize_rejects_nonfinite(oracle):
    x = np.ones((2, 8), dtype=np.float16)
    x[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_act(x, 0)


def test_int4_weight_quant(oracle):
    w = synth.weights(32, 256, seed=4)
    codes, s = oracle.quantize_weight_int4(w, 128)
    assert codes.min() >= -7 and codes.max() <= 7
    assert np.all(np.abs(codes.reshape(32, 2, 128)).max(axis=2) == 7)
    packed = oracle.pack_int4(codes)
    assert packed.shape == (32, 128)
    np.testing.assert_array_equal(oracle.unpack_int4(packed, 256), codes)
    # nibble layout: low nibble holds the even k
    lo = (packed & 0xF).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    np.testing.assert_array_equal(lo, codes[:, 0::2])
