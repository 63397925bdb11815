"""GPU parity of the int8 GEMMs: raw int32 sums and per-group partials bit for
bit, fp16 outputs within tolerance, against the oracle on the same seeded
int8 codes and scales (drawn by the input generator, not by either side).

Shapes are chosen to exercise every tile configuration the library selects
(32x32, 64x64, 64x128, 128x128, 128x160, 256x128, 256x160, 256x320, the few-token
row-range form with each of its token paddings 16/32/64/128, one or several
passes over a workgroup's rows, and workgroups with no K to do, and the
row-range form with shared stages for 33-256 tokens with one and two token
slices, one and two token blocks per wave, workgroups without rows and K
stages fewer than its ring holds), ragged M/N
edges, N not a multiple of 4 (scalar stores), and K with a half-filled last
stage (K % 128 == 64); test_tile_selection asserts which configuration the
shapes the tests rely on run (gemm_tile_config)."""
import numpy as np
import pytest

import synth
from tests.parity_util import assert_equal, assert_fp16_close, dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    return require_gpu()


# (M, N, K): covers the 32x128, 64x128, 128x128, 256x128 and 256x160 selections
PC_SHAPES = [
    (16, 512, 256), (1, 96, 64), (3, 100, 192), (64, 64, 64),
    (65, 130, 320), (200, 300, 192), (257, 321, 256),
    (1024, 4096, 128), (2048, 8192, 128), (2048, 10240, 128), (1500, 10240, 192),
    # ragged M and N (N not a multiple of 160), rows not a multiple of 16
    # bytes (scalar stores), few stages per tile, a K tail: 128x128 and
    # 256x128 tiles as the tile-cost model picks them
    (2000, 8200, 1024), (1800, 8196, 1280), (2048, 8192, 512), (2000, 8200, 320),
    (1500, 8196, 320), (1500, 8200, 1280),
    # 256x160 tiles, one round over the CUs, ragged M
    (1000, 10240, 256),
    # 256x320 tiles of eight waves: two tiles per workgroup, 8 K-stages (the
    # ring of two wraps four times per tile and the stage stream crosses
    # tile boundaries); then a ragged last tile row (4000 = 15 * 256 + 160)
    (4096, 10240, 1024), (4000, 10240, 640),
    # 128x160 tiles (one round where 256-row tiles leave compute units idle):
    # ragged M, a K tail
    (4000, 1280, 640), (3900, 1280, 704),
    # few tokens: 32x32 and 64x64 tiles, N ragged against them (scalar stores
    # where N % 8 != 0), a K tail; the M = 32 / 64 rows of the N=10240 K=2560
    # layer
    (32, 1000, 448), (31, 1030, 320), (48, 1030, 448), (33, 2051, 192),
    (32, 10240, 2560), (64, 10240, 2560),
    # few tokens with N large enough that each workgroup streams several
    # tiles (the four-stage ring across tile boundaries), with stages per
    # tile below and above the ring depth
    (8, 49160, 256), (8, 49152, 640), (40, 40968, 192),
    # the few-token row-range form: tokens padded to 16, 32, 64, 128; rows per
    # workgroup 8 (N=2048) to 40 (N=10240); N ragged against the 8-row units
    # and not a multiple of 4; a K tail; K = 64 (one 64-byte stage: three of
    # the four waves have none); K / 64 odd; N < 8; several passes per
    # workgroup (more rows than one pass holds: N=40000 at 24 tokens, and
    # N=49160 at 8 tokens below)
    (5, 10240, 2560), (17, 4099, 448), (33, 2048, 1024), (100, 8192, 2560),
    (128, 4096, 4096), (65, 6150, 320), (7, 5, 64), (128, 1030, 64), (20, 8190, 4160),
    (24, 40000, 192),
    # 1-4 tokens: the matrix-vector form, one shape per lane split (K / 16
    # chunks <= 64, 128, 160, 256, more), N ragged against its 16 or 4 rows
    # per workgroup; M * K at 65536 (last one on this path) and just above
    (2, 1001, 1024), (4, 333, 2048), (3, 10240, 2560), (1, 4099, 4096), (4, 777, 16384),
    (2, 5, 32768), (4, 129, 16448), (3, 4099, 14336), (4, 4096, 12288),
    # 33-256 tokens, the row-range form with shared stages: 33-48 tokens at
    # N > 8192 (N ragged against the 8-row units and not a multiple of 4,
    # three stages against a ring of eight), up to 128 tokens at N <= 8192
    # (two token slices), K >= 8192 up to 256 tokens (two blocks of 16 tokens
    # per wave), N = 129 (most workgroups have no rows)
    (33, 10240, 2560), (47, 10243, 384), (77, 3001, 1280), (128, 8192, 4096),
    (200, 1030, 8192), (256, 2000, 8192), (40, 129, 256),
    # ... up to 256 tokens at N <= 5120 (two slices of 80, N ragged), and
    # 65-127 tokens up to N = 10240 (two slices of 56); wide outputs: one
    # slice of two token blocks per wave (N=14336), eight row blocks of 16
    # per range (N ragged against the 8-row units)
    (160, 4100, 1280), (112, 10000, 640), (96, 14336, 1024), (200, 16380, 256),
    (120, 30000, 256),
]


def _shape(cfg):
    """The tile configuration proper (occupancy may differ between the builds
    of one tile for different epilogues)."""
    return cfg["bm"], cfg["bn"], cfg["waves"]


# (M, N, K) -> (tile rows, tile columns, waves) of the per-channel GEMM and its
# int32 export, for the shapes whose tile choice the tests rely on
EXPECTED_TILES = {
    (4096, 10240, 1024): (256, 320, 8),
    (4000, 10240, 640): (256, 320, 8),
    (4096, 10240, 2560): (256, 320, 8),
    (8192, 10240, 2560): (256, 320, 8),
    (1000, 10240, 256): (256, 160, 4),
    (1024, 10240, 2560): (256, 160, 4),
    (1500, 10240, 192): (256, 128, 4),     # K % 128 != 0; 2 rounds of 256x128 beat 256x160
    (2000, 8200, 1024): (128, 128, 4),     # N % 160 != 0
    (2048, 10240, 128): (256, 320, 8),     # one K-stage per tile
    (4096, 1280, 2560): (128, 160, 4),     # 256 tiles of 128x160: one round
    (4000, 1280, 640): (128, 160, 4),
    # few tokens: the row-range form (tokens padded to 16, rows of one pass)
    (5, 10240, 2560): (16, 48, 4),         # 40 rows per workgroup
    (32, 10240, 2560): (32, 48, 4),
    (8, 49160, 256): (16, 128, 4),         # 192 rows per workgroup: two passes
    (7, 5, 64): (16, 16, 4),
    (24, 40000, 192): (32, 128, 4),        # 160 rows per workgroup: two passes
    (65, 6150, 320): (128, 32, 4),         # K % 128 != 0: not the shared-stage form
    (64, 10240, 2560): (64, 48, 4),        # one slice, 40 rows per workgroup
    (128, 10240, 2560): (64, 80, 4),       # two slices of 64 tokens, 80 rows
    # 33-256 tokens, the row-range form with shared stages (the tokens of a
    # slice padded to 64 per block per wave, the rows of a range padded to 16)
    (33, 10240, 2560): (64, 48, 4),        # one slice, 40 rows per workgroup
    (100, 8192, 2560): (64, 64, 4),        # two slices of 50 tokens, 64 rows
    (128, 4096, 4096): (64, 32, 4),
    (128, 8192, 4096): (64, 64, 4),
    (77, 3001, 1280): (64, 32, 4),
    (200, 1030, 8192): (128, 16, 4),       # two slices of 100 tokens
    (256, 2000, 8192): (128, 16, 4),
    (40, 129, 256): (64, 16, 4),
    (160, 4100, 1280): (128, 48, 4),       # two slices of 80 tokens, 40 rows
    (112, 10000, 640): (64, 80, 4),        # two slices of 56 tokens, 80 rows
    (96, 14336, 4096): (128, 64, 4),       # one slice (two blocks of 16 per wave), 56 rows
    (96, 14336, 1024): (128, 64, 4),
    (200, 16380, 256): (128, 128, 4),      # two slices of 100 tokens, 128 rows
    (120, 30000, 256): (128, 128, 4),      # one slice, 120 rows of 30000 / 256 ranges
}


def test_tile_selection(torch_gpu):
    import w4a8_int8_gemm_amd as w
    for (M, N, K), want in EXPECTED_TILES.items():
        t = w.gemm_tile_config(w.GemmOp.GEMM_PC, M, N, K)
        assert _shape(t) == want, ((M, N, K), t)
        assert _shape(w.gemm_tile_config(w.GemmOp.GEMM_I32, M, N, K)) == want, (M, N, K)
    # two tiles per workgroup at 4096 x 10240 (256 compute units, one each)
    t = w.gemm_tile_config(w.GemmOp.GEMM_PC, 4096, 10240, 1024)
    assert t["tiles"] >= 2 * t["grid"], t
    # every per-group and W4A8 raw-sum export takes its product's tile
    for gs in (64, 128):
        for (M, N, K) in [(1024, 4096, 256), (2048, 8192, 256), (1800, 6100, 384),
                          (4096, 14336, 4096), (4516, 24576, 4096), (31, 1000, 384)]:
            assert (_shape(w.gemm_tile_config(w.GemmOp.GEMM_PG, M, N, K, gs)) ==
                    _shape(w.gemm_tile_config(w.GemmOp.PG_PARTIALS, M, N, K, gs))), (M, N, K, gs)
            if M > 4:   # 1-4 tokens: the W4A8 product takes its matrix-vector form
                assert (_shape(w.gemm_tile_config(w.GemmOp.GEMM_W4A8, M, N, K, gs)) ==
                        _shape(w.gemm_tile_config(w.GemmOp.W4A8_PARTIALS, M, N, K, gs))), (M, N, K, gs)


@pytest.mark.parametrize("M,N,K", PC_SHAPES)
def test_gemm_i32_and_pc(torch_gpu, oracle, M, N, K):
    import w4a8_int8_gemm_amd as w
    print(f"gemm pc M={M} N={N} K={K}", flush=True)
    seed = M + N + K
    xq, wq = synth.int8_codes(M, K, seed, 0), synth.int8_codes(N, K, seed, 1)
    sa, sw = synth.scales(M, 0, seed, 0, 3.0), synth.scales(N, 0, seed, 1)
    c_ref = oracle.gemm_i32(xq, wq)
    y_ref = oracle.epilogue_pc(c_ref, sa, sw)
    c = w.w8a8_gemm_i32(dev(xq), dev(wq))
    assert_equal(host(c), c_ref, "int32 sums")
    y = w.w8a8_gemm_pc(dev(xq), dev(sa), dev(wq), dev(sw))
    stats = assert_fp16_close(host(y), y_ref, what="fp16 y")
    # both sides round (nearly) the same value: almost every output is identical
    assert stats["exact_frac"] > 0.99, stats


# Few to a few hundred tokens at the N=10240, K=2560 layer with N made ragged
# (10243: not a multiple of 8 or 4), through every form the dispatch picks on
# the way: the few-token matrix-vector form of the fp16 product (1) and the
# K-split row-range form (the int32 export at 1; 5, 8), the shared-stage
# row-range form (33), 64x64 tiles (64) and 64x128 tiles (128, 200, 256); int32
# sums bit for bit and fp16 against the oracle.
@pytest.mark.parametrize("M", [1, 5, 8, 33, 64, 128, 200, 256])
def test_tokens_sweep_ragged_n(torch_gpu, oracle, M):
    import w4a8_int8_gemm_amd as w
    N, K = 10243, 2560
    print(f"gemm pc token sweep M={M} N={N} K={K}", flush=True)
    seed = 7 * M + 1
    xq, wq = synth.int8_codes(M, K, seed, 0), synth.int8_codes(N, K, seed, 1)
    sa, sw = synth.scales(M, 0, seed, 0, 3.0), synth.scales(N, 0, seed, 1)
    c_ref = oracle.gemm_i32(xq, wq)
    assert_equal(host(w.w8a8_gemm_i32(dev(xq), dev(wq))), c_ref, "int32 sums")
    y = w.w8a8_gemm_pc(dev(xq), dev(sa), dev(wq), dev(sw))
    stats = assert_fp16_close(host(y), oracle.epilogue_pc(c_ref, sa, sw), what="fp16 y")
    assert stats["exact_frac"] > 0.99, stats


# The last three reach the 256x128 two-waves-per-SIMD tiles (>= 384 tiles);
# 1800x6100 is ragged in both M and N, and K = 448 leaves a 64-wide K tail
# (gs = 64 only).
PG_SHAPES = [(16, 512, 256), (3, 100, 384), (200, 300, 640), (257, 321, 512),
             (70, 200, 320), (1024, 4096, 256), (2048, 8192, 256), (1800, 6100, 384),
             (1800, 6100, 448),
             # few tokens: 32x32 tiles, N ragged against them
             (31, 1000, 384), (32, 1030, 256)]


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", PG_SHAPES)
def test_gemm_pg(torch_gpu, oracle, M, N, K, gs):
    import w4a8_int8_gemm_amd as w
    if K % gs:
        pytest.skip("K not a multiple of gs")
    print(f"gemm pg M={M} N={N} K={K} gs={gs}", flush=True)
    seed = M * 3 + N + K + gs
    G = K // gs
    xq, wq = synth.int8_codes(M, K, seed, 0), synth.int8_codes(N, K, seed, 1)
    sa, sw = synth.scales(M, G, seed, 0, 3.0), synth.scales(N, G, seed, 1)
    p_ref = oracle.gemm_partials(xq, wq, gs)
    y_ref, t_ref = oracle.epilogue_pg(p_ref, sa, sw)
    p = w.w8a8_gemm_pg_partials(dev(xq), dev(wq), gs)
    assert_equal(host(p), p_ref, "per-group partials")
    y = w.w8a8_gemm_pg(dev(xq), dev(sa), dev(wq), dev(sw), gs)
    assert_fp16_close(host(y), y_ref, t_ref, G, what="fp16 y")


# 1-4 tokens take the W4A8 matrix-vector form: 4, 8 and 16 chunks per lane
# (one pass, or several over a row), N ragged against 16 rows per workgroup,
# M * K at 65536 and just above it (the GEMM again)
W4_FEW_SHAPES = [(1, 1001, 1024), (2, 333, 2048), (4, 4099, 4096), (3, 6144, 4096),
                 (2, 257, 12288), (4, 100, 16384), (4, 129, 16512)]


@pytest.mark.parametrize("gs", [64, 128])
@pytest.mark.parametrize("M,N,K", PG_SHAPES + W4_FEW_SHAPES)
def test_gemm_w4a8(torch_gpu, oracle, M, N, K, gs):
    import w4a8_int8_gemm_amd as w
    if K % gs:
        pytest.skip("K not a multiple of gs")
    print(f"gemm w4a8 M={M} N={N} K={K} gs={gs}", flush=True)
    seed = M * 5 + N + K + gs
    G = K // gs
    xq, w4 = synth.int8_codes(M, K, seed, 0), synth.packed_int4(N, K, seed, 1)
    sa, sw = synth.scales(M, 0, seed, 0, 3.0), synth.scales(N, G, seed, 1, 0.3)
    p_ref = oracle.gemm_partials(xq, oracle.unpack_int4(w4, K), gs)
    y_ref, t_ref = oracle.epilogue_w4a8(p_ref, sa, sw)
    p = w.w4a8_gemm_partials(dev(xq), dev(w4), gs)
    assert_equal(host(p), p_ref, "per-group partials")
    y = w.w4a8_gemm(dev(xq), dev(sa), dev(w4), dev(sw), gs)
    assert_fp16_close(host(y), y_ref, t_ref, G, what="fp16 y")


def test_int4_every_nibble(torch_gpu, oracle):
    """Rows of 0x88 (two -8 codes, which the quantizer never emits) and 0x77."""
    import w4a8_int8_gemm_amd as w
    M, N, K, gs = 64, 64, 256, 128
    w4 = synth.packed_int4(N, K, 1)
    w4[0, :] = 0x88
    w4[1, :] = 0x77
    xq = synth.int8_codes(M, K, 1)
    xq[0, :] = -127
    p_ref = oracle.gemm_partials(xq, oracle.unpack_int4(w4, K), gs)
    assert_equal(host(w.w4a8_gemm_partials(dev(xq), dev(w4), gs)), p_ref, "partials")


def test_extreme_int8_codes(torch_gpu, oracle):
    """All +-127 codes at K = 16384: sums reach 127^2 * K."""
    import w4a8_int8_gemm_amd as w
    M, N, K = 64, 64, 16384
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    wq = np.full((N, K), 127, np.int8)
    wq[::3] = -127
    c_ref = oracle.gemm_i32(xq, wq)
    assert int(np.abs(c_ref).max()) == 127 * 127 * K
    assert_equal(host(w.w8a8_gemm_i32(dev(xq), dev(wq))), c_ref, "int32 sums")


@pytest.mark.parametrize("M", [32, 40])
def test_largest_k_extreme_codes(torch_gpu, oracle, M):
    """K = 133120, the largest multiple of 64 the per-channel entry points
    accept (127^2 K < 2^31): all-+-127 codes put the int32 sums within 0.02 %
    of the int32 limit, through the int32 export and the fp16 epilogue (32
    tokens: the K-split row-range form; 40: the shared-stage one)."""
    import w4a8_int8_gemm_amd as w
    N, K = 64, 133120
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    wq = np.full((N, K), 127, np.int8)
    wq[::3] = -127
    c_ref = oracle.gemm_i32(xq, wq)
    assert int(np.abs(c_ref).max()) == 127 * 127 * K
    assert_equal(host(w.w8a8_gemm_i32(dev(xq), dev(wq))), c_ref, "int32 sums at the largest K")
    sa, sw = synth.scales(M, 0, 3, 0, 1e-6), synth.scales(N, 0, 3, 1, 1e-3)
    y = w.w8a8_gemm_pc(dev(xq), dev(sa), dev(wq), dev(sw))
    assert_fp16_close(host(y), oracle.epilogue_pc(c_ref, sa, sw), what="fp16 y at the largest K")


def test_zero_rows_and_empty(torch_gpu):
    import torch
    import w4a8_int8_gemm_amd as w
    M, N, K = 70, 96, 256
    xq, wq = synth.int8_codes(M, K, 1), synth.int8_codes(N, K, 2)
    xq[5] = 0
    sa, sw = synth.scales(M, 0, 1), synth.scales(N, 0, 2)
    y = host(w.w8a8_gemm_pc(dev(xq), dev(sa), dev(wq), dev(sw)))
    assert np.all(y[5] == 0)
    e = torch.empty((0, K), dtype=torch.int8, device="cuda")
    out = w.w8a8_gemm_pc(e, torch.empty((0,), dtype=torch.float32, device="cuda"), dev(wq), dev(sw))
    assert out.shape == (0, N)


def test_epilogue_rounds_to_nearest_even(torch_gpu, oracle):
    """With unit scales every output is fp16(an integer that fp32 holds exactly),
    so the result is fixed bit for bit; about one in eight outputs is an exact
    tie between two fp16 neighbours (round-toward-zero would miss those)."""
    import w4a8_int8_gemm_amd as w
    M, N, K = 128, 256, 256
    xq, wq = synth.int8_codes(M, K, 11, 0), synth.int8_codes(N, K, 11, 1)
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    c = oracle.gemm_i32(xq, wq)
    y_ref = oracle.epilogue_pc(c, ones_m, ones_n)
    y = host(w.w8a8_gemm_pc(dev(xq), dev(ones_m), dev(wq), dev(ones_n)))
    ties = np.abs(c) > 2048
    assert ties.mean() > 0.5
    assert_equal(y.view(np.uint16), y_ref.view(np.uint16), "fp16 bits (unit scales)")
    for gs in (64, 128):
        G = K // gs
        p = oracle.gemm_partials(xq, wq, gs)
        y_ref, _ = oracle.epilogue_pg(p, np.ones((M, G), np.float32), np.ones((N, G), np.float32))
        y = host(w.w8a8_gemm_pg(dev(xq), dev(np.ones((M, G), np.float32)), dev(wq),
                                dev(np.ones((N, G), np.float32)), gs))
        assert_equal(y.view(np.uint16), y_ref.view(np.uint16), f"pg gs={gs} fp16 bits")
        w4 = synth.packed_int4(N, K, 12)
        p = oracle.gemm_partials(xq, oracle.unpack_int4(w4, K), gs)
        y_ref, _ = oracle.epilogue_w4a8(p, ones_m, np.ones((N, G), np.float32))
        y = host(w.w4a8_gemm(dev(xq), dev(ones_m), dev(w4), dev(np.ones((N, G), np.float32)), gs))
        assert_equal(y.view(np.uint16), y_ref.view(np.uint16), f"w4a8 gs={gs} fp16 bits")
