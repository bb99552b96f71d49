"""Parity of every rung of the HIP ladder with the CPU oracle, through the
C ABI (tiling_roofline_analysis_amd's ctypes binding of libtra_gemm.so).

Acceptance:
  * integer-pattern and small-integer inputs: the GPU's C equals the oracle's
    C32 exactly (all partial sums are integers below 2^24, so every order of
    summation gives the same value; compared with ==, so +0 and -0 are equal);
  * floating-point inputs: |C_gpu - C64| <= 1e-5 * S per element, where C64
    is the oracle's binary64 sum and S = sum_k |A_ik * B_kj|.
Full-size shapes are checked on every element against the oracle's full
product, and on sampled entries the oracle computes one by one (whole rows
and columns at tile edges plus random entries); the integer patterns are
checked on every element through their period (C depends only on i mod 13
and j mod 7).
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import pytest

import oracle
import tiling_roofline_analysis_amd as tra
from tiling_roofline_analysis_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-5
# the four rungs of the ladder and the stream-K form of the MFMA rung
RUNGS = [tra.NAIVE, tra.LDS_TILED, tra.REGBLOCK_DB, tra.MFMA, tra.MFMA_STREAMK]
RUNG_IDS = ["naive", "lds_tiled", "regblock_db", "mfma", "mfma_streamk"]
C_SENTINEL = np.float32(12345.0)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tra.load()   # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def to_device(x: np.ndarray, ld: int, off: int, fill=np.nan):
    """Flat device buffer holding row-major x with leading dimension ld,
    starting `off` floats in; returns (tensor, address of x[0,0])."""
    import torch
    rows, cols = x.shape
    n = off + max(rows * ld, 1)
    host = np.full(n, np.float32(fill), np.float32)
    if rows and cols:
        host[off:off + rows * ld].reshape(rows, ld)[:, :cols] = x
    t = torch.from_numpy(host).to("cuda:0")
    return t, t.data_ptr() + 4 * off


def run_gpu(variant, A, B, lda=None, ldb=None, ldc=None, offs=(0, 0, 0), stream=None,
            c_init=C_SENTINEL):
    """C = A x B on the GPU; returns (C (M x N), whole C buffer, ldc, off)."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    tA, pA = to_device(A, lda, offs[0])
    tB, pB = to_device(B, ldb, offs[1])
    nC = offs[2] + max(M * ldc, 1)
    tC = torch.full((nC,), float(c_init), dtype=torch.float32, device="cuda:0")
    pC = tC.data_ptr() + 4 * offs[2]
    s = stream if stream is not None else torch.cuda.current_stream()
    st = tra.gemm_f32_variant(variant, M, N, K, pA, lda, pB, ldb, pC, ldc, s.cuda_stream)
    assert st == tra.TRA_OK, tra.tra_status_string(st)
    torch.cuda.synchronize()
    buf = tC.cpu().numpy()
    C = buf[offs[2]:offs[2] + M * ldc].reshape(M, ldc)[:, :N] if M else np.zeros((0, N), np.float32)
    return C, buf, ldc, offs[2]


def assert_exact(C, ref32, what):
    bad = C != ref32
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements differ; first at "
                           f"{np.argwhere(bad)[0]}: gpu {C[bad][0]} vs {ref32[bad][0]}")


def assert_tol(C, c64, s64, what):
    err = np.abs(C.astype(np.float64) - c64)
    lim = TOL * s64
    bad = err > lim
    ratio = float(np.max(err / np.where(s64 > 0, s64, 1.0))) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond 1e-5*S "
                           f"(max |diff|/S = {ratio:.3e})")
    return ratio


@functools.lru_cache(maxsize=None)
def workload_inputs(name):
    return inputs.WORKLOADS[name].make()


@functools.lru_cache(maxsize=None)
def int_inputs(M, N, K):
    return inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)


@functools.lru_cache(maxsize=None)
def oracle_full(name):
    A, B = workload_inputs(name)
    return oracle.gemm(A, B)


# --- the configured small shapes, every element -------------------------------

@pytest.mark.parametrize("name", ["int256", "const256", "int1024", "uniform1024"])
@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_small_configs_full(variant, name):
    log(f"[case] {tra.tra_gemm_variant_name(variant)} {name}")
    A, B = workload_inputs(name)
    ref = oracle_full(name)
    C, *_ = run_gpu(variant, A, B)
    w = inputs.WORKLOADS[name]
    if w.kind in ("int", "const"):
        # integer patterns are exact; the constant case is exact in the
        # oracle but not for every binary32 summation order
        if w.kind == "int":
            assert_exact(C, ref.c32, name)
        assert_tol(C, ref.c64, ref.s64, name)
    else:
        assert_tol(C, ref.c64, ref.s64, name)


def test_constant_256_close_to_51_2():
    A, B = workload_inputs("const256")
    for v in RUNGS:
        C, *_ = run_gpu(v, A, B)
        assert np.all(np.abs(C.astype(np.float64) - 51.20000076293945) <= TOL * 51.20000076293945)


# --- the configured large shapes ----------------------------------------------

def edge_indices(n, extra=()):
    cand = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 511, 512, n // 2, n - 2, n - 1, *extra}
    return sorted(i for i in cand if 0 <= i < n)


def sample_entries(M, N, seed, n_random=20000):
    rng = np.random.default_rng(seed)
    rs, cs = [], []
    for i in edge_indices(M)[:6] + edge_indices(M)[-3:]:
        rs.append(np.full(N, i))
        cs.append(np.arange(N))
    for j in edge_indices(N)[:6] + edge_indices(N)[-3:]:
        rs.append(np.arange(M))
        cs.append(np.full(M, j))
    rs.append(rng.integers(0, M, n_random))
    cs.append(rng.integers(0, N, n_random))
    return np.concatenate(rs), np.concatenate(cs)


# the configured large shapes, and one GPU's slab of the two largest split
# over 8 GPUs (512 rows of 4096^3; 2048 of the tall-skinny K)
LARGE = ["normal4096", "ragged", "tall", "rowslab4096", "kslab_tall"]


@pytest.mark.parametrize("name", LARGE)
@pytest.mark.parametrize("variant", RUNGS + [tra.AUTO], ids=RUNG_IDS + ["auto"])
def test_large_configs_every_element(variant, name):
    # every element against the oracle's full product (computed once per
    # configuration: about 20 s at 4096^3 on 16 cores), and a sample of
    # rows, columns and random entries computed directly, one by one
    w = inputs.WORKLOADS[name]
    log(f"[case] {tra.tra_gemm_variant_name(variant)} {name} {w.M}x{w.N}x{w.K} "
        f"({tra.tra_gemm_describe(variant, w.M, w.N, w.K)})")
    A, B = workload_inputs(name)
    C, *_ = run_gpu(variant, A, B)
    ref = oracle_full(name)
    ratio = assert_tol(C, ref.c64, ref.s64, name)
    log(f"[case]   every element within 1e-5 * S; max |diff|/S = {ratio:.2e}")
    rows, cols = sample_entries(w.M, w.N, seed=w.M)
    direct = oracle.gemm_entries(A, B, rows, cols)
    assert_tol(C[rows, cols], direct.c64, direct.s64, f"{name} (direct)")


@pytest.mark.parametrize("name", LARGE)
@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_large_shapes_int_patterns_every_element(variant, name):
    w = inputs.WORKLOADS[name]
    log(f"[case] int patterns {tra.tra_gemm_variant_name(variant)} {w.M}x{w.N}x{w.K}")
    A, B = int_inputs(w.M, w.N, w.K)
    C, *_ = run_gpu(variant, A, B)
    # the oracle's values on one period, then every element through it
    ii, jj = np.meshgrid(np.arange(min(13, w.M)), np.arange(min(7, w.N)), indexing="ij")
    per = oracle.gemm_entries(A, B, ii.ravel(), jj.ravel())
    T = per.c32.reshape(ii.shape)
    exp = T[np.arange(w.M)[:, None] % 13, np.arange(w.N)[None, :] % 7]
    assert_exact(C, exp, f"int patterns {name}")
    # and a sample directly from the oracle, not through the period
    rows, cols = sample_entries(w.M, w.N, seed=1, n_random=2000)
    direct = oracle.gemm_entries(A, B, rows, cols)
    assert_exact(C[rows, cols], direct.c32, f"int patterns {name} (direct)")


# --- tails, strides, alignment -------------------------------------------------

EDGE_M = [1, 17, 33, 65, 129, 257]
EDGE_K = [1, 2, 15, 16, 17, 31, 32, 33, 127, 129]


@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_edge_sizes(variant):
    rng = np.random.default_rng(21)
    for M in EDGE_M:
        for N in EDGE_M:
            for K in EDGE_K:
                A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
                B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
                ref = oracle.gemm(A, B)
                C, *_ = run_gpu(variant, A, B)
                assert_tol(C, ref.c64, ref.s64, f"{M}x{N}x{K}")
                Ai = inputs.small_ints(M, K, M * 1000 + K)
                Bi = inputs.small_ints(K, N, N * 1000 + K)
                refi = oracle.gemm(Ai, Bi)
                Ci, *_ = run_gpu(variant, Ai, Bi)
                assert_exact(Ci, refi.c32, f"small ints {M}x{N}x{K}")


# Every (M, N) pair of the tile-edge sizes, with K running through the same
# sizes, so that each size appears on each axis next to every other size.
EDGE_ALL = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 257]


@pytest.mark.parametrize("variant", RUNGS + [tra.AUTO], ids=RUNG_IDS + ["auto"])
def test_edge_sizes_all_pairs(variant):
    n = len(EDGE_ALL)
    for i, M in enumerate(EDGE_ALL):
        for j, N in enumerate(EDGE_ALL):
            K = EDGE_ALL[(i + 3 * j) % n]
            Ai = inputs.small_ints(M, K, 7 * M + K)
            Bi = inputs.small_ints(K, N, 11 * N + K)
            refi = oracle.gemm(Ai, Bi)
            Ci, *_ = run_gpu(variant, Ai, Bi)
            assert_exact(Ci, refi.c32, f"small ints {M}x{N}x{K}")


# Shapes that send the MFMA rung to each of its tile shapes, with tails on
# every axis and register-staged slices (K not a multiple of 4 where the
# 64 x 64 tiles would otherwise load directly into LDS): (M, N, K, expected
# tile).
MFMA_TILE_SHAPES = [
    (4000, 4200, 1027, "<256x128x16, 8 waves, 4 sets>"),   # 16 x 33 = 528 tiles of 256 x 128
    (1900, 2000, 300, "<128x128x16, 8 waves>"),   # 15 x 16 = 240 tiles of 128 x 128
    (1500, 1500, 77, "<64x64x16, 4 waves>"),      # 576 tiles of 64 x 64, short K
    (200, 300, 4101, "<64x64x16, 4 waves, 4 sets>"),   # few tiles, long K
    (300, 500, 203, "<64x64x16, 4 waves>"),       # few tiles
    (700, 900, 1501, "<64x64x16, 4 waves, 4 sets>"),   # 165 tiles, K > 1024
    (2040, 4090, 300, "<256x128x16, 8 waves, 4 sets>"),   # 8 x 32 = 256 tiles of 256 x 128
    (2000, 2600, 2050, "<128x128x16, 8 waves>"),  # 336 tiles of 128 x 128, K >= 2048
    (3000, 32, 1100, "<64x64x16, 4 waves, 4 sets>"),   # narrower than a tile (float4 loads)
    (40, 2000, 700, "<64x64x16, 4 waves>"),       # shorter than a tile (float4 loads)
    (3000, 33, 1100, "<64x64x16, 4 waves, 4 sets>"),   # narrower than a tile, N odd
    (200, 65500, 40, "<256x128x16, 8 waves, 4 sets>"),   # large tiles taller than M
    (100, 30001, 40, "<128x128x16, 8 waves>"),    # 128 x 128 tiles taller than M, N odd
]


@functools.lru_cache(maxsize=None)
def tile_shape_case(M, N, K):
    A = inputs.uniform(M, K, 77)
    B = inputs.uniform(K, N, 78)
    return A, B, oracle.gemm(A, B)


@pytest.mark.parametrize("shape", MFMA_TILE_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_tile_shapes_with_tails(variant, shape):
    M, N, K, tile = shape
    if variant in (tra.MFMA, tra.MFMA_STREAMK):
        assert tile in tra.tra_gemm_describe(variant, M, N, K)
    A, B, ref = tile_shape_case(M, N, K)
    C, *_ = run_gpu(variant, A, B)
    assert_tol(C, ref.c64, ref.s64, f"{M}x{N}x{K}")


# Shapes whose main launch stages its slices with direct loads into LDS
# (64 x 64 tiles, K a multiple of 16, 16-byte-aligned rows, every tile
# inside the matrices, at least twice as many slices as stages, no split),
# in both 64 x 64 tile classes, with M and N not multiples of the tile
# (edge tiles moved inside), at the fewest slices that take it and one more,
# and one tile alone: (M, N, K, kernel the MFMA rung plans).  The
# stream-K form of the same shapes runs register-staged.
# R below: the slices left for the unrolled last iterations (6 to 12)
_DMA = "<64x64x16, 4 waves, 6 LDS stages>"
DMA_SHAPES = [
    (1000, 1000, 1024, _DMA),     # R = 10
    (1000, 1000, 208, _DMA),      # 13 slices, the fewest; R = 7
    (1000, 1000, 224, _DMA),      # R = 8
    (1000, 1000, 528, _DMA),      # R = 9
    (64, 64, 560, _DMA),          # one tile, R = 11
    (700, 900, 1536, _DMA),       # R = 6
    (64, 64, 1040, _DMA),         # 65 slices, one tile
    (3000, 2052, 1536, _DMA),     # 1551 tiles
    (200, 300, 4112, _DMA),       # 20 tiles, long K
    # K a multiple of 4 but not of 16: the last slice runs past K
    (1000, 1000, 1000, _DMA),     # 8 of its 16 k inside, R = 9
    (1000, 1000, 516, _DMA),      # 4 inside
    (700, 900, 1548, _DMA),       # 12 inside, R = 7
    (64, 64, 1044, _DMA),         # one tile, R = 12
    (1000, 1000, 196, _DMA),      # 13 slices, R = 7
    (1000, 1000, 212, _DMA),      # R = 8
    (300, 500, 244, _DMA),        # R = 10
    (300, 500, 260, _DMA),        # R = 11
    (16384, 64, 4112, _DMA),      # one column of tiles, A 270 MB; R = 11
    (16384, 64, 4100, _DMA),      # 4 of the last slice's 16 k inside, R = 11
    (32768, 64, 1024, _DMA),      # 512 tiles in one column (128 x 128 tiles would be half outside)
]


@pytest.mark.parametrize("shape", DMA_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
@pytest.mark.parametrize("variant", [tra.MFMA, tra.MFMA_STREAMK, tra.AUTO],
                         ids=["mfma", "mfma_streamk", "auto"])
def test_direct_load_staging(variant, shape):
    M, N, K, kernel = shape
    assert f"kernel=gemm_mfma_f32{kernel} " in tra.tra_gemm_describe(tra.MFMA, M, N, K)
    log(f"[case] direct loads {tra.tra_gemm_variant_name(variant)} {M}x{N}x{K}")
    A, B, ref = tile_shape_case(M, N, K)
    C, *_ = run_gpu(variant, A, B)
    assert_tol(C, ref.c64, ref.s64, f"{M}x{N}x{K}")
    Ai = inputs.small_ints(M, K, 3 * M + K)
    Bi = inputs.small_ints(K, N, 5 * N + K)
    Ci, *_ = run_gpu(variant, Ai, Bi)
    assert_exact(Ci, oracle.gemm(Ai, Bi).c32, f"small ints {M}x{N}x{K}")


def test_direct_load_staging_with_padded_rows():
    # leading dimensions above the row length that keep rows 16-byte
    # aligned still take the direct loads; C's odd ldc is only stored to
    M, N, K = 1000, 1000, 1024
    A, B, ref = tile_shape_case(M, N, K)
    for variant in (tra.MFMA, tra.AUTO):
        log(f"[case] direct loads, padded rows, {tra.tra_gemm_variant_name(variant)}")
        C, buf, ldc, off = run_gpu(variant, A, B, lda=K + 12, ldb=N + 4, ldc=N + 3)
        assert_tol(C, ref.c64, ref.s64, "padded rows")
        pad = buf[off:off + M * ldc].reshape(M, ldc)[:, N:]
        assert (pad == C_SENTINEL).all(), "C written past its rows"


# Shapes that send the register-blocked rung to its K split inside the
# workgroup (4, 3 or 2 lane groups each running an equal share of the K
# slices), with tails on every axis: (M, N, K, lane groups).
REGBLOCK_SPLIT_SHAPES = [
    (1024, 1024, 1024, 4),   # the 1024^3 configuration: 256 tiles, 64 slices
    (1000, 1000, 1000, 3),   # 63 slices, the last one partial; edge tiles moved inside
    (1000, 1000, 1007, 3),   # K tail 15 of 16
    (300, 700, 255, 4),      # 16 slices, the last partial
    (100, 200, 127, 2),      # 8 slices
    (60, 50, 760, 4),        # one tile larger than the matrix (checked loads)
    (2048, 512, 1024, 4),    # 256 tiles, 2048 x 512
]


@pytest.mark.parametrize("shape", REGBLOCK_SPLIT_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_regblock_k_split(shape):
    M, N, K, groups = shape
    d = tra.tra_gemm_describe(tra.REGBLOCK_DB, M, N, K)
    log(f"[case] regblock K split {M}x{N}x{K} ({d})")
    assert f"K in {groups}>" in d
    A, B = inputs.uniform(M, K, 91), inputs.uniform(K, N, 92)
    ref = oracle.gemm(A, B)
    C, *_ = run_gpu(tra.REGBLOCK_DB, A, B)
    assert_tol(C, ref.c64, ref.s64, f"{M}x{N}x{K}")
    Ai, Bi = inputs.small_ints(M, K, M + 3), inputs.small_ints(K, N, N + 5)
    Ci, *_ = run_gpu(tra.REGBLOCK_DB, Ai, Bi)
    assert_exact(Ci, oracle.gemm(Ai, Bi).c32, f"small ints {M}x{N}x{K}")
    # odd strides and 4-byte offsets: element loads, element stores
    Cs, buf, ldc_, off = run_gpu(tra.REGBLOCK_DB, Ai, Bi, K + 3, N + 5, N + 7, (1, 3, 1))
    assert_exact(Cs, oracle.gemm(Ai, Bi).c32, f"odd strides {M}x{N}x{K}")
    full = buf[off:off + M * ldc_].reshape(M, ldc_)
    assert np.all(full[:, N:] == C_SENTINEL)


@functools.lru_cache(maxsize=None)
def stride_case(M, N, K):
    A = inputs.uniform(M, K, 5)
    B = inputs.uniform(K, N, 6)
    return A, B, oracle.gemm(A, B)


@pytest.mark.parametrize("layout", ["padded_aligned", "padded_misaligned"])
@pytest.mark.parametrize("shape", [(300, 200, 150), (4000, 4200, 1027), (1500, 1500, 77),
                                   (50, 36, 300)],
                         ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_strides_and_alignment(variant, shape, layout):
    M, N, K = shape

    def up4(x):
        return (x + 3) // 4 * 4

    if layout == "padded_aligned":     # vector-load path with padded rows
        lda, ldb, ldc, offs = up4(K) + 4, up4(N) + 8, up4(N) + 4, (0, 0, 0)
    else:                              # element-load path: odd strides, 4-byte offsets
        lda, ldb, ldc, offs = K + 3, N + 5, N + 7, (1, 3, 1)
    A, B, ref = stride_case(M, N, K)
    C, buf, ldc_, off = run_gpu(variant, A, B, lda, ldb, ldc, offs)
    assert_tol(C, ref.c64, ref.s64, f"{layout} {shape}")
    # nothing outside the first N columns of each row of C was written
    full = buf[off:off + M * ldc_].reshape(M, ldc_)
    assert np.all(full[:, N:] == C_SENTINEL)
    assert np.all(buf[:off] == C_SENTINEL)


# --- element offsets past 2^31 ------------------------------------------------
# Rows of 65536 floats: 40000 of them span 2.6e9 elements (10.5 GB), so the
# last rows of the strided operand start beyond element 2^31 (byte 2^33).
# An index or offset kept in 32 bits would read or write the wrong place.
HUGE_LD = 65536


def strided_on_device(x: np.ndarray, ld: int):
    """Device buffer of rows x ld floats holding x in its first columns, the
    four words after each row set to C_SENTINEL; returns (buffer, view)."""
    import torch
    rows, cols = x.shape
    buf = torch.empty(rows * ld, dtype=torch.float32, device="cuda:0")
    view = buf.view(rows, ld)
    view[:, cols:cols + 4].fill_(float(C_SENTINEL))
    view[:, :cols].copy_(torch.from_numpy(x))
    return buf, view


# The MFMA rung's full slices load through buffer resources at 32-bit byte
# offsets from the tile's corner; rows of A 2^23 floats apart (the 64 x 64
# tile's 64 rows span 2^31 bytes) or rows of B 2^25 apart are beyond that,
# and those launches load element by element instead.
@pytest.mark.parametrize("case", ["A_rows", "B_rows"])
@pytest.mark.parametrize("variant", [tra.MFMA, tra.MFMA_STREAMK, tra.AUTO],
                         ids=["mfma", "mfma_streamk", "auto"])
def test_rows_beyond_buffer_offsets(variant, case):
    import torch
    M, N, K = (130, 70, 300) if case == "A_rows" else (100, 70, 40)
    ld = (1 << 23) + 4 if case == "A_rows" else (1 << 25) + 4
    A, B = int_inputs(M, N, K)
    ref = oracle.gemm(A, B)
    log(f"rows beyond buffer offsets: {case} {M}x{N}x{K} ld {ld} variant {variant}")
    vC = torch.full((M, N), float(C_SENTINEL), dtype=torch.float32, device="cuda:0")
    if case == "A_rows":
        buf, v = strided_on_device(A, ld)
        other = torch.from_numpy(B).to("cuda:0")
        args = (v.data_ptr(), ld, other.data_ptr(), N, vC.data_ptr(), N)
    else:
        buf, v = strided_on_device(B, ld)
        other = torch.from_numpy(A).to("cuda:0")
        args = (other.data_ptr(), K, v.data_ptr(), ld, vC.data_ptr(), N)
    st = tra.gemm_f32_variant(variant, M, N, K, *args, torch.cuda.current_stream().cuda_stream)
    assert st == tra.TRA_OK, tra.tra_status_string(st)
    torch.cuda.synchronize()
    C = vC.cpu().numpy()
    del buf, v, other, vC
    torch.cuda.empty_cache()
    assert_exact(C, ref.c32, f"{case} variant {variant}")


@pytest.mark.parametrize("case", ["A_and_C_rows", "B_rows"])
@pytest.mark.parametrize("variant", RUNGS + [tra.AUTO], ids=RUNG_IDS + ["auto"])
def test_offsets_past_2_31_elements(variant, case):
    import torch
    # K = 512 (32 slices) and K = 40000: the MFMA rung's unsplit launches
    # stage these with direct loads into LDS, the split ones through
    # registers
    if case == "A_and_C_rows":
        M, N, K = 40000, 64, 512
    else:
        M, N, K = 64, 64, 40000
    A, B = int_inputs(M, N, K)
    ref = oracle.gemm(A, B)
    log(f"offsets past 2^31: {case} {M}x{N}x{K} variant {variant}")
    keep = []   # the device buffers, freed at the end
    if case == "A_and_C_rows":
        bufA, vA = strided_on_device(A, HUGE_LD)
        tB = torch.from_numpy(B).to("cuda:0")
        bufC, vC = strided_on_device(np.zeros((M, N), np.float32), HUGE_LD)
        vC[:, :N].fill_(float(C_SENTINEL))
        keep += [bufA, tB, bufC]
        args = (vA.data_ptr(), HUGE_LD, tB.data_ptr(), N, vC.data_ptr(), HUGE_LD)
        assert (M - 1) * HUGE_LD > 2 ** 31
    else:
        tA = torch.from_numpy(A).to("cuda:0")
        bufB, vB = strided_on_device(B, HUGE_LD)
        vC = torch.full((M, N), float(C_SENTINEL), dtype=torch.float32, device="cuda:0")
        keep += [tA, bufB, vC]
        args = (tA.data_ptr(), K, vB.data_ptr(), HUGE_LD, vC.data_ptr(), N)
        assert (K - 1) * HUGE_LD > 2 ** 31
    st = tra.gemm_f32_variant(variant, M, N, K, *args, torch.cuda.current_stream().cuda_stream)
    assert st == tra.TRA_OK, tra.tra_status_string(st)
    torch.cuda.synchronize()
    C = vC[:, :N].cpu().numpy()
    tail_ok = case != "A_and_C_rows" or bool(torch.all(vC[:, N:N + 4] == float(C_SENTINEL)))
    del keep, vC
    if case == "A_and_C_rows":
        del bufA, vA, bufC
    else:
        del bufB, vB
    torch.cuda.empty_cache()
    assert_exact(C, ref.c32, f"{case} variant {variant}")
    assert tail_ok, "a word after a row of C was written"


@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_k_zero_writes_zeros(variant):
    A = np.zeros((70, 0), np.float32)
    B = np.zeros((0, 130), np.float32)
    C, *_ = run_gpu(variant, A, B, lda=0, ldb=130, c_init=np.nan)
    assert np.all(C == 0.0)


@pytest.mark.parametrize("variant", RUNGS, ids=RUNG_IDS)
def test_empty_output_untouched(variant):
    import torch
    c = torch.full((16,), 7.0, device="cuda:0")
    assert tra.gemm_f32_variant(variant, 0, 4, 4, 0, 4, 0, 4, c.data_ptr(), 4, None) == tra.TRA_OK
    assert tra.gemm_f32_variant(variant, 4, 0, 4, 0, 4, 0, 4, c.data_ptr(), 4, None) == tra.TRA_OK
    torch.cuda.synchronize()
    assert torch.all(c == 7.0)


# --- cross-rung, determinism, streams, errors ----------------------------------

def test_rungs_agree_bitwise_on_int_patterns_1024():
    # every rung gives the same bits (the page reports max |diff| = 0 between
    # its naive and tiled kernels on these inputs)
    A, B = workload_inputs("int1024")
    outs = [run_gpu(v, A, B)[0] for v in RUNGS]
    for o in outs[1:]:
        assert float(np.max(np.abs(o - outs[0]))) == 0.0
    assert_exact(outs[0], oracle_full("int1024").c32, "int1024")


@pytest.mark.parametrize("name", ["uniform1024", "ragged"])
def test_mfma_deterministic(name):
    # bitwise the same over 10 runs, for each MFMA form (the stream-K partial
    # sums are added in a fixed K order, not in the order workgroups finish)
    A, B = workload_inputs(name)
    for variant in (tra.MFMA, tra.MFMA_STREAMK, tra.AUTO):
        first = run_gpu(variant, A, B)[0]
        for _ in range(9):
            again = run_gpu(variant, A, B)[0]
            assert np.array_equal(again.view(np.uint32), first.view(np.uint32)), variant


def test_auto_is_mfma():
    A, B = workload_inputs("uniform1024")
    a = run_gpu(tra.AUTO, A, B)[0]
    m = run_gpu(tra.MFMA, A, B)[0]
    assert np.array_equal(a.view(np.uint32), m.view(np.uint32))


def test_non_default_stream_and_torch_wrapper():
    import torch
    A, B = workload_inputs("uniform1024")
    ref = oracle_full("uniform1024")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dA = torch.from_numpy(A).to("cuda:0", non_blocking=False)
        dB = torch.from_numpy(B).to("cuda:0", non_blocking=False)
        C = tra.matmul(dA, dB)
    s.synchronize()
    assert_tol(C.cpu().numpy(), ref.c64, ref.s64, "side stream")


def test_invalid_call_leaves_c_untouched():
    import torch
    a = torch.ones((8, 8), device="cuda:0")
    b = torch.ones((8, 8), device="cuda:0")
    c = torch.full((8, 8), 3.0, device="cuda:0")
    st = tra.gemm_f32_variant(tra.MFMA, 8, 8, 8, a.data_ptr(), 7, b.data_ptr(), 8,
                              c.data_ptr(), 8, None)
    assert st == tra.TRA_ERR_INVALID_ARG
    st = tra.gemm_f32_variant(tra.MFMA, 8, 8, 8, a.data_ptr(), 8, b.data_ptr(), 8,
                              a.data_ptr(), 8, None)
    assert st == tra.TRA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(c == 3.0) and torch.all(a == 1.0)
    with pytest.raises(ValueError):
        tra.matmul(a[:, :7], b)       # inner dimensions differ


# --- seeded random shapes: every MFMA path against the oracle -----------------

def _random_shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        # sizes around the tile edges of every class, K across the slice edges
        M = int(rng.choice([rng.integers(1, 70), rng.integers(60, 300), rng.integers(250, 700)]))
        N = int(rng.choice([rng.integers(1, 70), rng.integers(60, 300), rng.integers(250, 700)]))
        K = int(rng.choice([rng.integers(1, 40), rng.integers(30, 300), rng.integers(900, 1300)]))
        aligned = bool(rng.integers(0, 2))
        out.append((M, N, K, aligned))
    return out


@pytest.mark.parametrize("variant", [tra.AUTO, tra.MFMA, tra.MFMA_STREAMK],
                         ids=["auto", "mfma", "mfma_streamk"])
def test_random_shapes_small_ints_exact(variant):
    """Seeded random shapes with tails on every axis, aligned and odd
    strides; small-integer inputs make every partial sum exact, so the GPU
    must equal the oracle bit for bit whatever the tile, split or order."""
    for M, N, K, aligned in _random_shapes(2024, 24):
        log(f"[case] {tra.tra_gemm_variant_name(variant)} {M}x{N}x{K} aligned={aligned} "
            f"({tra.tra_gemm_describe(variant, M, N, K)})")
        A = inputs.small_ints(M, K, M * 7919 + K)
        B = inputs.small_ints(K, N, N * 7919 + K + 1)
        ref = oracle.gemm(A, B)
        if aligned:
            lda, ldb, ldc, offs = (K + 3) // 4 * 4, (N + 3) // 4 * 4, (N + 3) // 4 * 4, (0, 0, 0)
        else:
            lda, ldb, ldc, offs = K + 1, N + 3, N + 2, (1, 2, 3)
        C, buf, ldc_, off = run_gpu(variant, A, B, lda, ldb, ldc, offs)
        assert_exact(C, ref.c32, f"{M}x{N}x{K} aligned={aligned}")
        full = buf[off:off + M * ldc_].reshape(M, ldc_)
        assert np.all(full[:, N:] == C_SENTINEL), "wrote past column N"


def _random_direct_load_shapes(seed, n):
    # shapes whose MFMA launch stages with direct loads: M, N >= 64, N a
    # multiple of 4, K with at least 13 slices (K <= 1024, or more than 64
    # slices), a multiple of 16 or only of 4 (the last slice running past
    # K); leading dimensions padded by whole quads, so rows stay 16-byte
    # aligned
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(64, 700))
        N = 4 * int(rng.integers(16, 175))
        K = 16 * int(rng.integers(13, 65) if i % 2 == 0 else rng.integers(65, 100))
        if i % 4 >= 2:
            K -= 4 * int(rng.integers(1, 4))   # the last slice runs past K
        pads = tuple(4 * int(x) for x in rng.integers(0, 3, size=3))
        out.append((M, N, K, pads))
    return out


@pytest.mark.parametrize("variant", [tra.AUTO, tra.MFMA], ids=["auto", "mfma"])
def test_random_direct_load_shapes_exact(variant):
    """Seeded random shapes through the direct-load K loop (both 64 x 64
    classes, edge tiles moved inside, padded rows): exact on small
    integers, and C untouched past column N."""
    for M, N, K, (pa, pb, pc) in _random_direct_load_shapes(77, 16):
        assert "LDS stages" in tra.tra_gemm_describe(tra.MFMA, M, N, K), (M, N, K)
        log(f"[case] direct loads {tra.tra_gemm_variant_name(variant)} {M}x{N}x{K} "
            f"pads {pa},{pb},{pc}")
        A = inputs.small_ints(M, K, M * 31 + K)
        B = inputs.small_ints(K, N, N * 31 + K + 1)
        ref = oracle.gemm(A, B)
        C, buf, ldc, off = run_gpu(variant, A, B, K + pa, N + pb, N + pc)
        assert_exact(C, ref.c32, f"{M}x{N}x{K}")
        full = buf[off:off + M * ldc].reshape(M, ldc)
        assert np.all(full[:, N:] == C_SENTINEL), "wrote past column N"


@pytest.mark.parametrize("shape", [(150, 130, 70), (300, 500, 203), (40, 2000, 64)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant", RUNGS + [tra.AUTO], ids=RUNG_IDS + ["auto"])
def test_non_finite_inputs_propagate(variant, shape):
    # IEEE propagation: an infinity or NaN in A or B reaches exactly the
    # elements of C whose sums use it (inf * 0 = NaN, inf + -inf = NaN); the
    # other terms are small integers, so every summation order gives the
    # oracle's value, and the zeros a kernel pads with never meet them
    M, N, K = shape
    A = inputs.small_ints(M, K, 11)
    B = inputs.small_ints(K, N, 12)
    A[3, 5], A[M - 1, K // 2], A[M // 2, K - 1] = np.inf, -np.inf, np.nan
    B[K // 3, 4], B[K - 1, N - 1] = np.inf, -np.inf
    ref = oracle.gemm(A, B).c32
    assert np.isnan(ref).any() and np.isinf(ref).any()
    C, *_ = run_gpu(variant, A, B)
    same = (C == ref) | (np.isnan(C) & np.isnan(ref))
    assert same.all(), f"{int((~same).sum())} elements differ; first at {np.argwhere(~same)[0]}"


def _random_large_shapes(seed, n):
    # sides drawn around each tile class's range: 64 x 64 tiles (900-3000),
    # 128 x 128 tiles (about one per CU, 1750-2050) and 256 x 128 tiles
    # (at least 4 of 128 x 128 per CU, 4100-4700; K above 1024, where they
    # are taken also when they leave a partial last wave)
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        lo, hi = [(900, 3000), (1750, 2050), (4100, 4700)][i % 3]
        klo, khi = (1030, 1500) if i % 3 == 2 else (40, 700)
        out.append((int(rng.integers(lo, hi)), int(rng.integers(lo, hi)),
                    int(rng.integers(klo, khi))))
    return out


def _picker_route_shapes(seed):
    # seeded shapes on each route of the tile-class choice, with the tile
    # each must take: short K with M >= 2048 (64 x 64); 256 x 128 tiles that
    # would leave a partial last wave with K <= 1024 (64 x 64); the same
    # with K > 1024 (256 x 128, split); exactly three 128 x 128 tiles a CU
    # with K >= 2048 (128 x 128); N of 64 to 70 under tall M, where wider
    # tiles would lie half outside (64 x 64)
    rng = np.random.default_rng(seed)
    r = lambda lo, hi: int(rng.integers(lo, hi))
    out = []
    for _ in range(2):
        out += [((r(2048, 5000), r(1000, 5000), r(40, 257)), "64x64x16"),
                ((r(4300, 4700), r(4300, 4700), r(300, 1025)), "64x64x16"),
                ((r(4300, 4700), r(4300, 4700), r(1100, 1400)), "256x128x16"),
                ((r(1985, 2049), r(6081, 6145), r(2048, 2300)), "128x128x16"),
                ((r(20000, 33000), r(64, 71), r(100, 400)), "64x64x16")]
    return out


@pytest.mark.parametrize("variant", [tra.AUTO, tra.MFMA, tra.MFMA_STREAMK],
                         ids=["auto", "mfma", "mfma_streamk"])
def test_picker_routes_int_patterns_exact(variant):
    """Seeded shapes on every route of the tile-class choice take the tile
    that route names, and every element matches the oracle's values on one
    period of the integer patterns (13 x 7), plus a direct sample."""
    for (M, N, K), tile in _picker_route_shapes(23):
        d = tra.tra_gemm_describe(variant, M, N, K)
        log(f"[case] picker route {tra.tra_gemm_variant_name(variant)} {M}x{N}x{K} ({d})")
        assert f"tile={tile} " in d, (M, N, K, d)
        A, B = int_inputs(M, N, K)
        C, *_ = run_gpu(variant, A, B)
        ii, jj = np.meshgrid(np.arange(13), np.arange(7), indexing="ij")
        T = oracle.gemm_entries(A, B, ii.ravel(), jj.ravel()).c32.reshape(ii.shape)
        assert_exact(C, T[np.arange(M)[:, None] % 13, np.arange(N)[None, :] % 7],
                     f"{M}x{N}x{K}")
        rows, cols = sample_entries(M, N, seed=M + N, n_random=500)
        assert_exact(C[rows, cols], oracle.gemm_entries(A, B, rows, cols).c32,
                     f"{M}x{N}x{K} (direct)")


@pytest.mark.parametrize("variant", [tra.AUTO, tra.MFMA, tra.MFMA_STREAMK],
                         ids=["auto", "mfma", "mfma_streamk"])
def test_random_large_shapes_int_patterns_exact(variant):
    """Seeded random shapes large enough for every tile class and both forms
    of the K split (parts and stream-K runs), with tails on every axis; on
    the integer patterns C has period 13 x 7, so every element is checked
    against the oracle's values on one period, plus a direct sample."""
    for M, N, K in _random_large_shapes(11, 12):
        log(f"[case] int patterns {tra.tra_gemm_variant_name(variant)} {M}x{N}x{K} "
            f"({tra.tra_gemm_describe(variant, M, N, K)})")
        A, B = int_inputs(M, N, K)
        C, *_ = run_gpu(variant, A, B)
        ii, jj = np.meshgrid(np.arange(13), np.arange(7), indexing="ij")
        T = oracle.gemm_entries(A, B, ii.ravel(), jj.ravel()).c32.reshape(ii.shape)
        assert_exact(C, T[np.arange(M)[:, None] % 13, np.arange(N)[None, :] % 7],
                     f"{M}x{N}x{K}")
        rows, cols = sample_entries(M, N, seed=M + N, n_random=500)
        assert_exact(C[rows, cols], oracle.gemm_entries(A, B, rows, cols).c32,
                     f"{M}x{N}x{K} (direct)")
