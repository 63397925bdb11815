"""The Python binding rejects malformed arguments before anything reaches the
C ABI (no GPU needed).

The C entry points receive bare pointers: a scale vector of the wrong length,
a per-channel scale passed to a per-group call, a host tensor or a tensor of
the wrong dtype would make a kernel read past a buffer or read host memory.
The wrappers check every tensor's device, dtype and exact shape against the
operands.  Here the accepted device type is switched to "cpu" so that CPU
tensors pass the device check and the shape/dtype checks are what decide;
each case must raise before any kernel launch is attempted."""
import pytest

torch = pytest.importorskip("torch")

import w4a8_int8_gemm_amd as w  # noqa: E402
from w4a8_int8_gemm_amd import ops  # noqa: E402

M, N, K, GS = 8, 16, 256, 128
G = K // GS
# what the binding's own checks say (a failure anywhere later, e.g. at the
# device context, would not match)
CHECK = r"scale|group_size|K=|shape|workspace|must be|does not match|dims"


@pytest.fixture
def cpu_ok(monkeypatch):
    monkeypatch.setattr(ops, "_DEVICE_TYPE", "cpu")


def i8(*shape):
    return torch.zeros(shape, dtype=torch.int8)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.ones(shape, dtype=torch.float32)


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def test_host_tensors_rejected_without_override():
    with pytest.raises(ValueError, match="device tensor"):
        w.w8a8_gemm_pc(i8(M, K), f32(M), i8(N, K), f32(N))
    with pytest.raises(ValueError, match="device tensor"):
        w.linear(w.Mode.W8A8_PC, f16(M, K), i8(N, K), f32(N))


@pytest.mark.parametrize("xs,ws,exc", [
    (f32(M + 1), f32(N), ValueError),            # token scales too long
    (f32(M), f32(N - 1), ValueError),            # channel scales too short
    (f32(M, 1), f32(N), ValueError),             # wrong rank
    (f32(M), f32(N, G), ValueError),             # per-group scales to a per-channel call
    (f32(M).half(), f32(N), TypeError),          # fp16 scales
    (f32(M), f32(N).double(), TypeError),        # fp64 scales
])
def test_gemm_pc_scales(cpu_ok, xs, ws, exc):
    with pytest.raises(exc, match=CHECK):
        w.w8a8_gemm_pc(i8(M, K), xs, i8(N, K), ws)


@pytest.mark.parametrize("xs,ws,gs", [
    (f32(M, G), f32(N), GS),                     # per-channel scales to a per-group call
    (f32(M), f32(N, G), GS),                     # per-token activation scales
    (f32(M, G + 1), f32(N, G), GS),              # one group too many
    (f32(M, G), f32(N, G), 96),                  # unsupported group size
    (f32(M, K // 64), f32(N, K // 64), 192),     # group size that is not 64/128
])
def test_gemm_pg_scales(cpu_ok, xs, ws, gs):
    with pytest.raises(ValueError, match=CHECK):
        w.w8a8_gemm_pg(i8(M, K), xs, i8(N, K), ws, gs)


@pytest.mark.parametrize("xs,ws", [
    (f32(M), f32(N)),                            # per-channel weight scales
    (f32(M, G), f32(N, G)),                      # per-group activation scales
    (f32(M), f32(N, G - 1)),                     # one group short
])
def test_gemm_w4a8_scales(cpu_ok, xs, ws):
    with pytest.raises(ValueError, match=CHECK):
        w.w4a8_gemm(i8(M, K), xs, u8(N, K // 2), ws, GS)


def test_weight_shape_and_dtype(cpu_ok):
    with pytest.raises(ValueError, match=CHECK):
        w.w8a8_gemm_pc(i8(M, K), f32(M), i8(N, K + 64), f32(N))     # K mismatch
    with pytest.raises(TypeError, match=CHECK):
        w.w8a8_gemm_pc(i8(M, K), f32(M), u8(N, K), f32(N))          # packed weights to int8 call
    with pytest.raises(ValueError, match=CHECK):
        w.w4a8_gemm(i8(M, K), f32(M), u8(N, K), f32(N, G), GS)      # unpacked width


def test_device_mismatch(cpu_ok):
    meta = torch.empty((N,), dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match=CHECK):
        w.w8a8_gemm_pc(i8(M, K), f32(M), i8(N, K), meta)


@pytest.mark.parametrize("mode,wt,ws,gs", [
    (w.Mode.W8A8_PG, i8(N, K), f32(N), GS),      # per-channel scales with the per-group mode
    (w.Mode.W8A8_PC, i8(N, K), f32(N, G), 0),    # per-group scales with the per-channel mode
    (w.Mode.W4A8, u8(N, K // 2), f32(N), GS),    # per-channel scales with int4 weights
    (w.Mode.W4A8, i8(N, K), f32(N, G), GS),      # int8 weights with the int4 mode
    (w.Mode.W8A8_PG, i8(N, K), f32(N, G), 100),  # bad group size
])
def test_linear_scales(cpu_ok, mode, wt, ws, gs):
    with pytest.raises((ValueError, TypeError), match=CHECK):
        w.linear(mode, f16(M, K), wt, ws, gs)


def test_linear_workspace(cpu_ok):
    need = w.linear_workspace_size(w.Mode.W8A8_PC, M, K)
    assert need > 0
    with pytest.raises(ValueError, match=CHECK):
        w.linear(w.Mode.W8A8_PC, f16(M, K), i8(N, K), f32(N), workspace=u8(need - 1))
    with pytest.raises(TypeError, match=CHECK):
        w.linear(w.Mode.W8A8_PC, f16(M, K), i8(N, K), f32(N), workspace=i8(need))


def test_decode_scales(cpu_ok):
    with pytest.raises(ValueError, match=CHECK):
        w.int8_mv(f16(K), i8(N, K), f32(N - 1))
    with pytest.raises(ValueError, match=CHECK):
        w.w8a8_mv_pg(f16(K), i8(N, K), f32(N), GS)
    with pytest.raises(ValueError, match=CHECK):
        w.w4a8_mv(f16(K), u8(N, K // 2), f32(N, G + 1), GS)


def test_comparison_gemm_scales(cpu_ok):
    with pytest.raises(ValueError, match=CHECK):
        w.w8a16_gemm(f16(M, K), i8(N, K), f32(N, 1))
    with pytest.raises(ValueError, match=CHECK):
        w.w4a16_gemm(f16(M, K), u8(N, K // 2), f32(N), GS)


def test_partials_group_size(cpu_ok):
    with pytest.raises(ValueError, match=CHECK):
        w.w8a8_gemm_pg_partials(i8(M, K), i8(N, K), 96)
    with pytest.raises(ValueError, match=CHECK):
        w.w4a8_gemm_partials(i8(M, K), u8(N, K // 2), 0)


def test_valid_arguments_pass_the_checks(cpu_ok):
    """Well-formed arguments get past every check: the first failure is the
    device context (host tensors cannot be launched on), not a check."""
    with pytest.raises(Exception) as e:
        w.w8a8_gemm_pg(i8(M, K), f32(M, G), i8(N, K), f32(N, G), GS)
    assert not isinstance(e.value, (TypeError,)) and "must" not in str(e.value), e.value
    with pytest.raises(Exception) as e:
        w.linear(w.Mode.W4A8, f16(M, K), u8(N, K // 2), f32(N, G), GS)
    assert "must" not in str(e.value) and "shape" not in str(e.value), e.value
