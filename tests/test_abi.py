"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import w4a8_int8_gemm_amd as w

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

P = ctypes.c_void_p
A = P(4096)          # a 16-byte aligned stand-in address; never dereferenced by these calls
A2 = P(8192)
A3 = P(12288)
A4 = P(16384)
A5 = P(20480)
MIS = P(4098)        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ["quantize_act", "w8a8_gemm_pc", "w8a8_gemm_pg", "w4a8_gemm", "int8_mv", "linear",
               "quantize_weight_int8", "pack_weight_int4", "w4a8_is_available",
               "w4a8_status_string", "w4a8_last_error", "linear_workspace_size",
               "w8a8_gemm_i32", "w8a8_gemm_pg_partials", "w4a8_gemm_partials",
               "w8a8_mv_pg", "w4a8_mv"]:
        assert fn in names, fn


def test_library_exports_every_declared_symbol():
    L = w.lib()
    for fn in declared_functions():
        assert hasattr(L, fn), f"libw4a8.so does not export {fn}"
    # and the binding wraps each with the same name
    for fn in declared_functions():
        if not fn.startswith("w4a8_"):
            assert hasattr(w, fn), f"binding lacks {fn}"


def test_exports_are_c_symbols():
    # extern "C": no C++ mangling on the public names
    out = os.popen(f"nm -D --defined-only {w.LIB_PATH}").read()
    for fn in declared_functions():
        assert re.search(rf"\sT\s{fn}$", out, flags=re.M), fn


def test_status_strings():
    L = w.lib()
    for s in w.Status:
        assert L.w4a8_status_string(int(s)).decode()
    assert L.w4a8_status_string(99) == b"unknown status"


def _last():
    return w.lib().w4a8_last_error().decode()


@pytest.mark.parametrize("call,status", [
    # quantize_act(x, M, K, gs, xq, xs, stream)
    (lambda L: L.quantize_act(A, 4, 12, 0, A2, A3, None), w.Status.ERR_SHAPE),
    (lambda L: L.quantize_act(A, 4, 0, 0, A2, A3, None), w.Status.ERR_SHAPE),
    (lambda L: L.quantize_act(A, -1, 16, 0, A2, A3, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.quantize_act(A, 4, 256, 32, A2, A3, None), w.Status.ERR_SHAPE),
    (lambda L: L.quantize_act(A, 4, 192, 128, A2, A3, None), w.Status.ERR_SHAPE),
    (lambda L: L.quantize_act(None, 4, 256, 0, A2, A3, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.quantize_act(MIS, 4, 256, 0, A2, A3, None), w.Status.ERR_ALIGNMENT),
    (lambda L: L.quantize_act(None, 0, 256, 0, None, None, None), w.Status.OK),
    (lambda L: L.pack_weight_int4(A, 4, 256, 0, A2, A3, None), w.Status.ERR_SHAPE),
    # w8a8_gemm_pc(xq, sa, wq, sw, y, M, N, K, stream)
    (lambda L: L.w8a8_gemm_pc(A, A2, A3, A4, A5, 4, 8, 96, None), w.Status.ERR_SHAPE),
    (lambda L: L.w8a8_gemm_pc(A, A2, A3, A4, A5, 4, 8, 133248, None), w.Status.ERR_SHAPE),
    (lambda L: L.w8a8_gemm_pc(A, None, A3, A4, A5, 4, 8, 128, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.w8a8_gemm_pc(A, A2, MIS, A4, A5, 4, 8, 128, None), w.Status.ERR_ALIGNMENT),
    (lambda L: L.w8a8_gemm_pc(None, None, None, None, None, 0, 8, 128, None), w.Status.OK),
    (lambda L: L.w8a8_gemm_pc(None, None, None, None, None, 4, 0, 128, None), w.Status.OK),
    # w8a8_gemm_pg(xq, sa, wq, sw, gs, y, M, N, K, stream)
    (lambda L: L.w8a8_gemm_pg(A, A2, A3, A4, 32, A5, 4, 8, 256, None), w.Status.ERR_SHAPE),
    (lambda L: L.w8a8_gemm_pg(A, A2, A3, A4, 128, A5, 4, 8, 320, None), w.Status.ERR_SHAPE),
    (lambda L: L.w4a8_gemm(A, A2, A3, A4, 0, A5, 4, 8, 256, None), w.Status.ERR_SHAPE),
    # int8_mv(x, wq, sw, y, N, K, xq_out, xs_out, stream)
    (lambda L: L.int8_mv(A, A2, A3, A4, 8, 24, None, None, None), w.Status.ERR_SHAPE),
    (lambda L: L.int8_mv(A, A2, A3, A4, 8, 32784, None, None, None), w.Status.ERR_SHAPE),
    (lambda L: L.int8_mv(None, A2, A3, A4, 8, 64, None, None, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.int8_mv(A, A2, A3, A4, 0, 64, None, None, None), w.Status.OK),
    # w8a8_mv_pg / w4a8_mv(x, w, sw, gs, y, N, K, stream)
    (lambda L: L.w8a8_mv_pg(A, A2, A3, 32, A4, 8, 256, None), w.Status.ERR_SHAPE),
    (lambda L: L.w8a8_mv_pg(A, A2, A3, 128, A4, 8, 320, None), w.Status.ERR_SHAPE),
    (lambda L: L.w8a8_mv_pg(A, A2, A3, 64, A4, 8, 32832, None), w.Status.ERR_SHAPE),
    (lambda L: L.w8a8_mv_pg(None, A2, A3, 64, A4, 8, 256, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.w8a8_mv_pg(A, None, A3, 64, A4, 8, 256, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.w8a8_mv_pg(A, MIS, A3, 64, A4, 8, 256, None), w.Status.ERR_ALIGNMENT),
    (lambda L: L.w8a8_mv_pg(A, A2, A3, 64, A4, 0, 256, None), w.Status.OK),
    (lambda L: L.w4a8_mv(A, A2, A3, 0, A4, 8, 256, None), w.Status.ERR_SHAPE),
    (lambda L: L.w4a8_mv(A, A2, A3, 128, A4, 8, 192, None), w.Status.ERR_SHAPE),
    (lambda L: L.w4a8_mv(MIS, A2, A3, 128, A4, 8, 256, None), w.Status.ERR_ALIGNMENT),
    (lambda L: L.w4a8_mv(A, A2, A3, 128, A4, -1, 256, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.w4a8_mv(A, A2, A3, 128, A4, 0, 256, None), w.Status.OK),
    # linear(mode, x, M, K, w, sw, gs, N, y, ws, ws_bytes, stream)
    (lambda L: L.linear(7, A, 4, 256, A2, A3, 0, 8, A4, A5, 1 << 20, None), w.Status.ERR_INVALID_ARG),
    (lambda L: L.linear(0, A, 4, 256, A2, A3, 0, 8, A4, None, 0, None), w.Status.ERR_WORKSPACE),
    (lambda L: L.linear(0, A, 4, 256, A2, A3, 0, 8, A4, A5, 16, None), w.Status.ERR_WORKSPACE),
    (lambda L: L.linear(0, A, 4, 256, A2, A3, 0, 8, A4, P(4096 + 16), 1 << 20, None), w.Status.ERR_WORKSPACE),
    (lambda L: L.linear(1, A, 4, 256, A2, A3, 48, 8, A4, A5, 1 << 20, None), w.Status.ERR_SHAPE),
    (lambda L: L.linear(0, A, 0, 256, A2, A3, 0, 8, A4, None, 0, None), w.Status.OK),
])
def test_argument_errors_before_device(call, status):
    L = w.lib()
    got = call(L)
    assert got == int(status), (got, status, _last())
    if status != w.Status.OK:
        assert _last()


def test_workspace_size():
    L = w.lib()
    a256 = lambda v: (v + 255) // 256 * 256
    assert L.linear_workspace_size(0, 4096, 2560, 0) == a256(4096 * 2560) + a256(4096 * 4)
    assert L.linear_workspace_size(1, 4096, 4096, 64) == a256(4096 * 4096) + a256(4096 * 64 * 4)
    assert L.linear_workspace_size(2, 4516, 4096, 128) == a256(4516 * 4096) + a256(4516 * 4)
    assert L.linear_workspace_size(0, 1, 2560, 0) == 0
    assert L.linear_workspace_size(1, 1, 4096, 128) == 0      # decode: matrix-vector kernels
    assert L.linear_workspace_size(2, 1, 4096, 64) == 0
    assert L.linear_workspace_size(1, 1, 65536, 128) == a256(65536) + a256(512 * 4)
    assert L.linear_workspace_size(0, 0, 2560, 0) == 0


def test_valid_call_without_gpu_reports_device():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = w.lib()
    assert L.w4a8_is_available() == 0
    assert L.quantize_act(A, 4, 256, 0, A2, A3, None) == int(w.Status.ERR_DEVICE)
    assert "device" in _last()
    with pytest.raises(w.W4A8Error):
        w.check(L.w8a8_gemm_pc(A, A2, A3, A4, A5, 4, 8, 128, None))
