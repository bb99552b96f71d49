"""Parity through the LDS-poison test build of the library.

libtra_gemm_poison.so is the same source built with TRA_LDS_POISON=1: every
kernel that stages operands in LDS fills its LDS with NaN before first use.
A kernel that reads an LDS word no lane staged -- a wrong index, a padding
word, a slice read before it was stored -- then puts NaN into C.  On small
integer inputs every correct order of summation gives the same bits, so the
check is exact equality with the CPU oracle on shapes that reach every tile
class, load mode and tail of every rung.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
import tiling_roofline_analysis_amd as tra
from tiling_roofline_analysis_amd import inputs

pytestmark = pytest.mark.gpu

VARIANTS = [tra.NAIVE, tra.LDS_TILED, tra.REGBLOCK_DB, tra.MFMA, tra.MFMA_STREAMK, tra.AUTO]
VARIANT_IDS = ["naive", "lds_tiled", "regblock_db", "mfma", "mfma_streamk", "auto"]
SHAPES = [
    (1, 1, 1), (17, 33, 15), (65, 129, 31), (129, 257, 33), (257, 65, 129),
    (300, 500, 203),      # few 64 x 64 tiles (stream-K shares all of them)
    (1500, 1500, 77),     # short K
    (200, 300, 4100),     # few tiles, long K
    (700, 900, 1500),     # 64 x 64, four register sets
    (1900, 2000, 300),    # 128 x 128 tiles
    (4000, 4200, 1027),    # 256 x 128 tiles, every edge ragged
    (2040, 4090, 300),    # 256 tiles of 256 x 128
    (2000, 2600, 2050),   # 128 x 128 with stream-K
    (3000, 2049, 1531),   # the ragged configuration
    (3000, 32, 1100),     # narrower than a tile: float4 loads, column quads past N zeroed
    (40, 2000, 700),      # shorter than a tile: float4 loads, rows past M zeroed
    (3000, 33, 1100),     # narrower than a tile, N odd: element loads
    (200, 65500, 40),     # 256 x 128 tiles taller than M
    (1000, 1000, 1007),   # register-blocked rung: K split over 3 lane groups, K tail
    (300, 700, 255),      # register-blocked rung: K split over 4 lane groups
    (100, 200, 127),      # register-blocked rung: K split over 2 lane groups
    (1000, 1000, 528),    # direct loads into LDS, 64 x 64, K <= 1024
    (700, 900, 1536),     # direct loads, K > 1024
    (64, 64, 1040),       # direct loads, one tile
    (200, 300, 4112),     # direct loads, few tiles, long K
    (1000, 1000, 208),    # direct loads, the fewest slices (13)
    (1000, 1000, 1000),   # direct loads, the last slice past K
    (700, 900, 1548),     # direct loads, the last slice past K
    (300, 500, 260),      # direct loads, the last slice past K, 17 slices
    (16384, 64, 4112),    # direct loads, one column of tiles, long K
    (16384, 64, 4100),    # the same, the last slice past K
]


@functools.lru_cache(maxsize=None)
def case(M, N, K):
    A = inputs.small_ints(M, K, 3 * M + K)
    B = inputs.small_ints(K, N, 5 * N + K)
    return A, B, oracle.gemm(A, B).c32


@pytest.fixture(scope="module")
def plib():
    return tra.load_poisoned()


def run(lib, variant, A, B):
    import torch
    M, K = A.shape
    N = B.shape[1]
    dA = torch.from_numpy(A).to("cuda:0")
    dB = torch.from_numpy(B).to("cuda:0")
    dC = torch.full((M, N), 12345.0, dtype=torch.float32, device="cuda:0")
    st = lib.gemm_f32_variant(variant, M, N, K, dA.data_ptr(), K, dB.data_ptr(), N,
                              dC.data_ptr(), N, torch.cuda.current_stream().cuda_stream)
    assert st == tra.TRA_OK, tra.tra_status_string(st)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_poisoned_build_exact(plib, variant, shape):
    M, N, K = shape
    print(f"[case] poison {tra.tra_gemm_variant_name(variant)} {M}x{N}x{K}", flush=True)
    A, B, ref = case(M, N, K)
    C = run(plib, variant, A, B)
    assert np.isfinite(C).all(), "NaN from an LDS word that no lane staged"
    bad = C != ref
    assert not bad.any(), f"{int(bad.sum())} elements differ"
