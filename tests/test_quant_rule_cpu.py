"""The GPU kernels' quantizer fast path (multiply by fl32(1/s), guard near
rounding boundaries, division rule for guarded elements) compiled for the
host and checked against the oracle on every fp16 input for many scales."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quant_rule_shim.cpp")


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("shim") / "quant_rule_shim.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", SRC, "-o", so, "-lm"], check=True)
    L = ctypes.CDLL(so)
    fp = ctypes.POINTER(ctypes.c_float)
    i8p = ctypes.POINTER(ctypes.c_int8)
    L.shim_quantize.argtypes = [fp, ctypes.c_int, ctypes.c_float, ctypes.c_float, i8p, fp]
    L.shim_quantize.restype = ctypes.c_int
    L.shim_fast_only.argtypes = [fp, ctypes.c_int, ctypes.c_float, ctypes.c_float, i8p]
    ip = ctypes.POINTER(ctypes.c_int)
    L.shim_check_corrected.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float, ip, ip]
    L.shim_check_corrected.restype = ctypes.c_long
    L.shim_count_uncorrected.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float]
    L.shim_count_uncorrected.restype = ctypes.c_long
    L.shim_check_scale.argtypes = [ctypes.c_float]
    L.shim_check_scale.restype = ctypes.c_long
    return L


def _run(shim, xs16: np.ndarray, amax16, qmax):
    x = xs16.astype(np.float32)
    q = np.empty(x.shape, np.int8)
    s = np.empty(1, np.float32)
    nslow = shim.shim_quantize(x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), x.size,
                               float(np.float32(amax16)), float(qmax),
                               q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)),
                               s.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return q, s[0], nslow


@pytest.mark.parametrize("qmax", [127, 7])
def test_fast_path_matches_oracle_exhaustively(shim, oracle, qmax):
    rng = np.random.default_rng(17)
    # 160 scales spread over the whole fp16 range, plus the edges
    amax_bits = np.unique(np.concatenate([
        rng.integers(0x0001, 0x7BFF, size=160), [0x0001, 0x03FF, 0x0400, 0x3C00, 0x57F0, 0x7BFF]
    ])).astype(np.uint16)
    total_slow = 0
    for ab in amax_bits.tolist():
        pos = np.arange(0, ab + 1, dtype=np.uint16)
        xs = np.concatenate([pos, pos | 0x8000]).view(np.float16)
        row = np.concatenate([[np.uint16(ab).view(np.float16)], xs])[None, :]
        want_q, want_s = oracle.quantize(row, 0, qmax)
        got_q, got_s, nslow = _run(shim, row[0], row[0, 0], qmax)
        total_slow += nslow
        assert got_s == want_s[0]
        np.testing.assert_array_equal(got_q, want_q[0], err_msg=f"amax bits {ab:#06x}")
    # the guard is rare: well under 0.1 % of elements take the division rule
    assert total_slow > 0


def test_guard_is_needed(shim, oracle):
    """Without the guard the reciprocal shortcut does disagree somewhere --
    so the exhaustive test above is a real check of the guard."""
    rng = np.random.default_rng(3)
    mismatches = 0
    for ab in rng.integers(0x0400, 0x7BFF, size=200).tolist():
        pos = np.arange(0, ab + 1, dtype=np.uint16)
        row = np.concatenate([[ab], pos]).astype(np.uint16).view(np.float16)[None, :]
        want_q, _ = oracle.quantize(row, 0, 127)
        x = row[0].astype(np.float32)
        q = np.empty(x.shape, np.int8)
        shim.shim_fast_only(x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), x.size,
                            float(x[0]), 127.0, q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)))
        mismatches += int((q != want_q[0]).sum())
        if mismatches:
            break
    assert mismatches > 0


@pytest.mark.parametrize("qmax", [127, 7])
def test_corrected_quotient_on_the_whole_domain(shim, qmax):
    """The kernels' division-free quotient for guarded elements (reciprocal,
    product, exact residual by fma, one correction) equals fl32(x / s) -- and
    its code the division rule's -- for every fp16 amax (s = fl32(amax/qmax))
    and every fp16 x with |x| <= amax, both signs: about 10^9 pairs, split
    over threads (each ctypes call releases the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    # ranges of amax bits with about equal work (work grows with the bits)
    top = 0x7C00
    edges = [1]
    for i in range(1, 64):
        edges.append(int(top * (i / 64) ** 0.5))
    edges.append(top)
    edges = sorted(set(edges))

    def run(k):
        a, b = ctypes.c_int(-1), ctypes.c_int(-1)
        n = shim.shim_check_corrected(edges[k], edges[k + 1], float(qmax), ctypes.byref(a),
                                      ctypes.byref(b))
        return n, a.value, b.value

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(run, range(len(edges) - 1)))
    bad = [(n, a, b) for n, a, b in results if n]
    assert not bad, f"mismatches (count, first amax bits, first x bits): {bad[:3]}"


def test_correction_step_is_needed(shim):
    """Without the correction the product fl32(x r) misses fl32(x / s) on
    part of the same domain, so the check above is a real one."""
    assert shim.shim_count_uncorrected(0x3C00, 0x3C40, 127.0) > 0


@pytest.mark.parametrize("qmax", [127, 7])
def test_scale_without_division_on_every_amax(shim, qmax):
    """The kernels' scale (reciprocal of qmax, product, one fma correction)
    equals fl32(amax / qmax) bit for bit for every non-negative fp16 amax."""
    assert shim.shim_check_scale(float(qmax)) == 0
