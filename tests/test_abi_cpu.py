"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-side argument checks reject bad calls before anything
is enqueued (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import numpy as np
import pytest

import tiling_roofline_analysis_amd as tra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tra_gemm.h")


def header_functions():
    text = open(HEADER).read()
    return re.findall(r"TRA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    return tra.load()


def test_header_declares_the_abi():
    names = header_functions()
    assert set(names) == set(tra.ABI_FUNCTIONS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("path", [tra.LIB_PATH, tra.POISON_LIB_PATH], ids=["product", "poison"])
def test_only_abi_symbols_are_exported(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    ours = {s for s in syms if not s.startswith("_")}
    assert ours == set(tra.ABI_FUNCTIONS), ours


def test_poison_library_loads_with_every_declared_symbol():
    plib = tra.load_poisoned()
    for name in header_functions():
        assert hasattr(plib, name), name
    assert plib is not tra.load()


def test_status_and_variant_names():
    assert tra.tra_status_string(tra.TRA_OK) == "ok"
    assert tra.tra_status_string(tra.TRA_ERR_INVALID_ARG) == "invalid argument"
    assert tra.tra_status_string(99) == "unknown"
    for name, v in tra.VARIANTS.items():
        assert tra.tra_gemm_variant_name(v) == name
    assert tra.tra_gemm_variant_name(-1) == "unknown"


def test_describe_plans():
    # the 8-wave tiles: register-staged slices in two LDS buffers
    d = tra.tra_gemm_describe(tra.MFMA, 4096, 4096, 4096)
    assert "gemm_mfma_f32" in d and "tile=256x128x16" in d and "grid=512" in d
    assert "block=512" in d and "4 sets" in d and "lds_bytes=57856" in d
    d = tra.tra_gemm_describe(tra.MFMA, 2048, 2048, 2048)
    assert "tile=128x128x16" in d and "8 waves" in d and "grid=256" in d and "block=512" in d
    # the 64 x 64 tiles with K a multiple of 16 and aligned rows: direct
    # loads into 6 LDS stages of 8448 bytes
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 1024)
    assert "tile=64x64x16" in d and "6 LDS stages" in d and "grid=256" in d and "block=256" in d
    assert "lds_bytes=50688" in d
    d = tra.tra_gemm_describe(tra.MFMA, 16384, 64, 16384)
    assert "tile=64x64x16" in d and "6 LDS stages" in d and "grid=256" in d
    assert "lds_bytes=50688" in d
    # K not a multiple of 4: register-staged slices, two LDS buffers
    d = tra.tra_gemm_describe(tra.MFMA, 3000, 2049, 1531)
    assert "tile=64x64x16" in d and "4 sets" in d and "grid=1551" in d and "block=256" in d
    assert "lds_bytes=18944" in d
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 1002)
    assert "<64x64x16, 4 waves>" in d and "lds_bytes=18944" in d
    # K a multiple of 4 but not of 16: direct loads, the last slice checked
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 1000)
    assert "6 LDS stages" in d and "lds_bytes=50688" in d
    # fewer than the 13 slices (2 x 6 + 1) the direct-load loop needs:
    # register-staged
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 192)
    assert "<64x64x16, 4 waves>" in d and "lds_bytes=18944" in d
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 208)
    assert "6 LDS stages" in d
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 196)    # 13 slices, the last past K
    assert "6 LDS stages" in d
    # direct loads address a lane's quad by a byte offset from the tile's
    # corner below 2^31: 64 rows of A 2^23 floats apart (lda = K) are too far
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, 1 << 23)
    assert "<64x64x16, 4 waves, 4 sets>" in d
    d = tra.tra_gemm_describe(tra.MFMA, 1024, 1024, (1 << 23) - 4)
    assert "6 LDS stages" in d
    d = tra.tra_gemm_describe(tra.NAIVE, 1024, 1024, 1024)
    assert "gemm_naive_f32" in d and "grid=4096" in d and "block=256" in d
    d = tra.tra_gemm_describe(tra.LDS_TILED, 1024, 1024, 1024)
    assert "tile=16x16x64" in d and "block=256" in d and "grid=4096" in d
    assert "lds_bytes=8704" in d
    d = tra.tra_gemm_describe(tra.REGBLOCK_DB, 3000, 2049, 1531)
    assert "grid=1551" in d and "64x64" in d    # 408 tiles of 128 x 128 are too few
    d = tra.tra_gemm_describe(tra.REGBLOCK_DB, 4096, 4096, 4096)
    assert "grid=1024" in d and "128x128" in d  # 4 tiles of 128 x 128 a CU
    d = tra.tra_gemm_describe(tra.REGBLOCK_DB, 3072, 3072, 3072)
    assert "grid=2304" in d and "64x64" in d    # 576 large tiles: 2.25 a CU
    assert tra.tra_gemm_describe(tra.AUTO, 16, 16, 16).startswith("variant=auto")
    # split in parts: 1551 tiles of 64 x 64 on 256 CUs x 3 workgroups leave
    # a last wave of 15 tiles, each cut into 8 parts of 12 slices that run in
    # the main launch (1551 + 15 x 7 workgroups), one partial tile of 16 KiB
    # per part
    d = tra.tra_gemm_describe(tra.MFMA_STREAMK, 3000, 2049, 1531)
    assert "stream_k_tiles=15" in d and "stream_k_wgs=120" in d
    assert "workspace_bytes=1966080" in d and "grid=1656" in d
    # whole waves of tiles: no split, no workspace
    d = tra.tra_gemm_describe(tra.MFMA_STREAMK, 4096, 4096, 4096)
    assert "stream_k_tiles=0" in d and "workspace_bytes=0" in d
    # fewer tiles than a wave: all of them split, 40 tiles x 13 slices into
    # 6 parts each (at least 2 slices a part)
    d = tra.tra_gemm_describe(tra.MFMA_STREAMK, 300, 500, 203)
    assert "stream_k_tiles=40" in d and "stream_k_wgs=240" in d and "grid=240" in d
    # stream-K runs: 648 tiles of 256 x 128 on 256 CUs leave 136, more than
    # half a wave, so their 136 x 256 slices go to 256 workgroups of 136
    # slices crossing tiles, two partial tiles of 128 KiB per workgroup; the
    # main launch adds 16 fixup chunks per shared tile (648 + 136 x 15)
    d = tra.tra_gemm_describe(tra.MFMA_STREAMK, 4608, 4608, 4096)
    assert "stream_k_tiles=136" in d and "stream_k_wgs=256" in d
    assert "workspace_bytes=67108864" in d and "grid=2688" in d
    assert "stream_k_tiles=0" in tra.tra_gemm_describe(tra.MFMA, 3000, 2049, 1531)
    with pytest.raises(tra.TraError):
        tra.tra_gemm_describe(7, 1, 1, 1)
    with pytest.raises(tra.TraError):
        tra.tra_gemm_describe(tra.MFMA, -1, 1, 1)


# Fake, never-dereferenced device addresses: the checks reject these calls on
# the host, before any HIP call.
A_ADDR, B_ADDR, C_ADDR = 0x10000000, 0x20000000, 0x30000000
INVALID = [
    # (variant, M, N, K, A, lda, B, ldb, C, ldc)
    (tra.MFMA, -1, 4, 4, A_ADDR, 4, B_ADDR, 4, C_ADDR, 4),          # negative M
    (tra.MFMA, 4, -1, 4, A_ADDR, 4, B_ADDR, 4, C_ADDR, 4),          # negative N
    (tra.MFMA, 4, 4, -1, A_ADDR, 4, B_ADDR, 4, C_ADDR, 4),          # negative K
    (tra.MFMA, 4, 4, 4, None, 4, B_ADDR, 4, C_ADDR, 4),             # A NULL
    (tra.MFMA, 4, 4, 4, A_ADDR, 4, None, 4, C_ADDR, 4),             # B NULL
    (tra.MFMA, 4, 4, 4, A_ADDR, 4, B_ADDR, 4, None, 4),             # C NULL
    (tra.MFMA, 4, 4, 8, A_ADDR, 7, B_ADDR, 4, C_ADDR, 4),           # lda < K
    (tra.MFMA, 4, 8, 4, A_ADDR, 4, B_ADDR, 7, C_ADDR, 8),           # ldb < N
    (tra.MFMA, 4, 8, 4, A_ADDR, 4, B_ADDR, 8, C_ADDR, 7),           # ldc < N
    (tra.MFMA, 4, 4, 4, A_ADDR, 4, B_ADDR, 4, A_ADDR + 16, 4),      # C overlaps A
    (tra.MFMA, 4, 4, 4, A_ADDR, 4, B_ADDR, 4, B_ADDR + 60, 4),      # C overlaps B's last word
    (tra.NAIVE, 4, 4, 4, A_ADDR, 4, B_ADDR, 4, B_ADDR - 4, 4),      # C's last word on B's first
    (6, 4, 4, 4, A_ADDR, 4, B_ADDR, 4, C_ADDR, 4),                  # unknown variant
    (-1, 4, 4, 4, A_ADDR, 4, B_ADDR, 4, C_ADDR, 4),                 # unknown variant
    (tra.MFMA, 1 << 40, 4, 4, A_ADDR, 1 << 40, B_ADDR, 4, C_ADDR, 4),   # extent overflow
]


@pytest.mark.parametrize("args", INVALID)
def test_invalid_arguments_rejected_on_host(args):
    v, M, N, K, A, lda, B, ldb, C, ldc = args
    st = tra.gemm_f32_variant(v, M, N, K, A, lda, B, ldb, C, ldc, None)
    assert st == tra.TRA_ERR_INVALID_ARG


def test_gemm_f32_checks_too():
    assert tra.gemm_f32(4, 4, 4, None, 4, B_ADDR, 4, C_ADDR, 4, None) == tra.TRA_ERR_INVALID_ARG


def test_grid_too_large_is_unsupported():
    # 2^36 rows x 64 columns of C with the naive rung needs 2^34 workgroups
    M = 1 << 36
    st = tra.gemm_f32_variant(tra.NAIVE, M, 64, 0, None, 0, None, 64, C_ADDR, 64, None)
    assert st == tra.TRA_ERR_UNSUPPORTED


def test_lane_count_past_32_bits_is_unsupported():
    # HIP needs grid x block below 2^32 in the x dimension: the naive rung
    # (256 lanes a workgroup) at 2^26 x 64 needs 2^24 workgroups, under the
    # workgroup limit but 2^32 lanes
    M = 1 << 26
    assert "grid=16777216 block=256" in tra.tra_gemm_describe(tra.NAIVE, M, 64, 0)
    st = tra.gemm_f32_variant(tra.NAIVE, M, 64, 0, None, 0, None, 64, C_ADDR, 64, None)
    assert st == tra.TRA_ERR_UNSUPPORTED


def test_noalloc_refuses_splits_past_its_scratch():
    # the stream-K runs of 4608^2 x 4096 need two 256 x 128 partial tiles for
    # each of 256 workgroups, 64 MiB, past the 32 MiB static scratch: refused
    # on the host, before anything is enqueued (nothing here touches a GPU)
    need = tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 4608, 4608, 4096)
    assert need == 64 << 20 > tra.STATIC_SCRATCH_BYTES
    st = tra.gemm_f32_variant_noalloc(tra.MFMA_STREAMK, 4608, 4608, 4096, A_ADDR, 4096, B_ADDR,
                                      4608, C_ADDR, 4608, None)
    assert st == tra.TRA_ERR_UNSUPPORTED
    # argument checks come first, as in gemm_f32_variant
    assert tra.gemm_f32_variant_noalloc(tra.MFMA, 4, 4, 4, None, 4, B_ADDR, 4, C_ADDR, 4,
                                        None) == tra.TRA_ERR_INVALID_ARG
    assert tra.gemm_f32_variant_noalloc(tra.MFMA, 0, 4, 4, None, 4, None, 4, None, 4,
                                        None) == tra.TRA_OK
    # the header's constant and the binding's agree
    text = open(HEADER).read()
    assert "#define TRA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)" in text


def test_release_without_workspaces_touches_nothing():
    # nothing was allocated in this process: OK without any HIP call
    assert tra.tra_gemm_release_workspaces() == tra.TRA_OK


@pytest.mark.parametrize("M,N", [(0, 5), (5, 0), (0, 0)])
def test_empty_output_is_noop(M, N):
    # nothing to compute: OK without touching any pointer (all NULL here)
    assert tra.gemm_f32_variant(tra.MFMA, M, N, 7, None, 7, None, 5, None, 5, None) == tra.TRA_OK


def test_probe_work_formulas():
    assert tra.tra_probe_work(tra.PROBE_COPY, 1000) == 8000.0
    # blocks x 4 waves x iters x 4 MFMAs x (2*32*32*2) flops
    assert tra.tra_probe_work(tra.PROBE_MFMA, 10) == 1024 * 4 * 10 * 4 * 4096
    # lanes x iters x 8 chains x 2 flops
    assert tra.tra_probe_work(tra.PROBE_FMA, 10) == 1024 * 256 * 10 * 8 * 2
    assert tra.tra_probe_work(9, 10) == -1.0
    assert tra.tra_probe_work(tra.PROBE_COPY, -1) == -1.0


def test_probe_invalid_arguments_rejected_on_host():
    bad = tra.TRA_ERR_INVALID_ARG
    assert tra.tra_probe_copy_f32(-1, A_ADDR, B_ADDR, None) == bad
    assert tra.tra_probe_copy_f32(16, None, B_ADDR, None) == bad
    assert tra.tra_probe_copy_f32(16, A_ADDR + 4, B_ADDR, None) == bad     # misaligned
    assert tra.tra_probe_copy_f32(16, A_ADDR, A_ADDR + 32, None) == bad    # overlap
    assert tra.tra_probe_copy_f32(0, None, None, None) == tra.TRA_OK
    assert tra.tra_probe_launch(0, None) == bad
    assert tra.tra_probe_launch(-3, None) == bad
    assert tra.tra_probe_launch(1 << 24, None) == bad      # 2^32 lanes, one too many
    assert tra.tra_probe_mfma_f32(-1, C_ADDR, None) == bad
    assert tra.tra_probe_mfma_f32(1, None, None) == bad
    assert tra.tra_probe_fma_f32(-1, C_ADDR, None) == bad
    assert tra.tra_probe_fma_f32(1, None, None) == bad


def test_python_matmul_rejects_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        tra.matmul(torch.zeros(2, 2), torch.zeros(2, 2))


def test_python_layout_check():
    # the leading dimension the binding passes for a view, or a refusal for
    # a view that is not row-major
    import torch
    base = torch.zeros(4, 8)
    ld = tra._row_major_ld
    assert ld(tuple(base.shape), base.stride(), "A") == 8
    assert ld(tuple(base[1:3, 2:7].shape), base[1:3, 2:7].stride(), "A") == 8
    assert ld(tuple(base[:1].shape), base[:1].stride(), "A") == 8
    assert ld(tuple(base[:, :1].shape), base[:, :1].stride(), "A") == 8
    assert ld((0, 5), (5, 1), "A") == 5
    # one row with every other element: not contiguous, refused (it used to
    # be passed as a dense row of 4)
    v = base[:1, ::2]
    assert tuple(v.shape) == (1, 4) and v.stride() == (8, 2)
    with pytest.raises(ValueError, match="unit column stride"):
        ld(tuple(v.shape), v.stride(), "A")
    with pytest.raises(ValueError, match="unit column stride"):
        ld(tuple(base.t().shape), base.t().stride(), "B")
    # rows that overlap (a broadcast view) are refused too
    e = torch.zeros(1, 3).expand(4, 3)
    with pytest.raises(ValueError, match="row stride"):
        ld(tuple(e.shape), e.stride(), "C")
    e1 = torch.zeros(1, 1).expand(4, 1)
    with pytest.raises(ValueError, match="row stride"):
        ld(tuple(e1.shape), e1.stride(), "C")


def test_workspace_size():
    assert tra.tra_gemm_workspace_size(tra.MFMA, 3000, 2049, 1531) == 0
    assert tra.tra_gemm_workspace_size(tra.NAIVE, 3000, 2049, 1531) == 0
    # one partial tile per part (120 parts of 64 x 64), or two per stream-K
    # workgroup (256 workgroups of 256 x 128 tiles)
    assert tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 3000, 2049, 1531) == 120 * 64 * 64 * 4
    assert (tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 4608, 4608, 4096)
            == 2 * 256 * 256 * 128 * 4)
    assert tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 4096, 4096, 4096) == 0
    assert tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 0, 2049, 1531) == 0
    # K of one slice (16 deep) leaves nothing to split
    assert tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 3000, 2049, 16) == 0
    for bad in [(6, 1, 1, 1), (tra.MFMA, -1, 1, 1), (tra.MFMA, 1, 1, -1)]:
        with pytest.raises(tra.TraError):
            tra.tra_gemm_workspace_size(*bad)
    out = ctypes.c_size_t(0)
    assert tra.load().tra_gemm_workspace_size(tra.MFMA, 1, 1, 1, None) == tra.TRA_ERR_INVALID_ARG


def test_caller_workspace_checked_on_host():
    M, N, K = 3000, 2049, 1531
    A, B, C = 0x100000000, 0x200000000, 0x300000000
    need = tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, M, N, K)
    ws = 0x400000000
    call = lambda w, n: tra.gemm_f32_variant_ws(tra.MFMA_STREAMK, M, N, K, A, K, B, N, C, N,
                                                w, n, None)
    assert call(None, need) == tra.TRA_ERR_INVALID_ARG       # needed but NULL
    assert call(ws, need - 1) == tra.TRA_ERR_INVALID_ARG     # too small
    assert call(ws + 4, need) == tra.TRA_ERR_INVALID_ARG     # not 16-byte aligned
    # the ordinary argument checks apply too
    assert tra.gemm_f32_variant_ws(tra.MFMA_STREAMK, M, N, K, None, K, B, N, C, N, ws, need,
                                   None) == tra.TRA_ERR_INVALID_ARG
    assert tra.gemm_f32_variant_ws(6, M, N, K, A, K, B, N, C, N, ws, need,
                                   None) == tra.TRA_ERR_INVALID_ARG
    # nothing to compute: OK with no workspace
    assert tra.gemm_f32_variant_ws(tra.MFMA_STREAMK, 0, N, K, None, K, None, N, None, N, None,
                                   0, None) == tra.TRA_OK


@pytest.mark.parametrize("shape,rung", [
    ((1024, 1024, 1024), "mfma"),          # 256 tiles on 256 CUs
    ((4096, 4096, 4096), "mfma"),          # 1024 tiles, 4 a CU
    ((3000, 2049, 1531), "mfma_streamk"),  # 1551 tiles: 6.06 a CU
    ((4608, 4608, 4096), "mfma_streamk"),  # 648 tiles of 256 x 128: 2.53 a CU
    ((3072, 3072, 3072), "mfma"),          # 2304 tiles: 9 a CU
    ((3008, 2048, 1536), "mfma"),          # 1504 tiles: 5.875 a CU, 2% short
    ((1500, 1500, 77), "mfma"),            # 3 slices of K: nothing to share
    ((1152, 1152, 8192), "mfma_streamk"),  # 324 tiles of one workgroup a CU
    ((16384, 64, 16384), "mfma"),          # 256 tiles
    ((200, 300, 4100), "mfma_streamk"),    # 20 tiles, 129 slices each
    ((300, 500, 203), "mfma"),             # 40 tiles of 7 slices: too short to share
    ((100, 100, 300), "mfma"),             # 4 tiles of 10 slices: saves < 8 us
    ((100, 100, 2000), "mfma_streamk"),    # 4 tiles of 63 slices
    ((3000, 3000, 1000), "mfma"),          # 2209 tiles: 8.63 a CU, 4.3% uneven
    ((2560, 3328, 1000), "mfma_streamk"),  # 2080 tiles: 8.13 a CU, 10.8% uneven (parts)
    ((2688, 2752, 1000), "mfma"),          # 1806 tiles: 13.4% uneven, but in stream-K runs
    ((3500, 3500, 1500), "mfma"),          # 3025 tiles: 11.82 a CU, 1.6% uneven
    ((5000, 5000, 1000), "mfma"),          # 800 tiles of 256 x 128 would be 3.13 a CU: 64 x 64 instead
    ((5880, 3806, 5236), "mfma_streamk"),  # 690 tiles of 256 x 128: 11.3% uneven (runs)
    ((6144, 3840, 4096), "mfma"),          # 720 tiles of 256 x 128: 6.7% uneven
    ((2560, 3072, 2048), "mfma"),          # 480 tiles of 128 x 128: 6.7% uneven
    ((8192, 64, 2048), "mfma_streamk"),    # 128 tiles: exactly half the CUs
    ((4096, 128, 2048), "mfma_streamk"),   # 128 tiles
    ((12288, 64, 2048), "mfma"),           # 192 tiles of 128 slices: saves < 8 us
    ((768, 768, 1024), "mfma"),            # 144 tiles of 64 slices: saves < 8 us
])
def test_auto_choice(shape, rung):
    d = tra.tra_gemm_describe(tra.AUTO, *shape)
    assert f"rung={rung} " in d, d


@pytest.mark.parametrize("shape,tile", [
    ((1024, 1024, 1024), "<64x64x16, 4 waves, 6 LDS stages>"),     # K <= 1024
    ((3000, 2049, 1531), "<64x64x16, 4 waves, 4 sets>"),    # 128x128 would waste the edge
    ((4096, 4096, 4096), "<256x128x16, 8 waves, 4 sets>"),  # 4 tiles of 128x128 a CU
    ((4096, 2048, 1024), "<256x128x16, 8 waves, 4 sets>"),  # exactly 256 tiles of 256x128
    ((2048, 4096, 2048), "<256x128x16, 8 waves, 4 sets>"),
    ((2048, 2048, 2048), "<128x128x16, 8 waves>"),          # one 128x128 tile a CU
    ((2304, 2304, 2304), "<128x128x16, 8 waves>"),          # 324 tiles, long K: parts
    ((2000, 2600, 3000), "<128x128x16, 8 waves>"),          # 336 tiles, edges wasted no worse
    ((3000, 3000, 1000), "<64x64x16, 4 waves, 6 LDS stages>"),     # short K stays on 64x64
    ((3072, 3072, 3072), "<64x64x16, 4 waves, 6 LDS stages>"),     # 576 tiles: 2.25 a CU
    # 256 tiles of 128x128 or 256x128 whose columns or rows lie half or
    # more outside the matrix: 64x64 tiles instead
    ((32768, 64, 8192), "<64x64x16, 4 waves, 6 LDS stages>"),
    ((65536, 64, 1024), "<64x64x16, 4 waves, 6 LDS stages>"),
    ((64, 65536, 4096), "<64x64x16, 4 waves, 6 LDS stages>"),
    ((384, 16384, 4096), "<128x128x16, 8 waves>"),  # not 256x128: a quarter outside
    ((2049, 32768, 1024), "<64x64x16, 4 waves, 6 LDS stages>"),
    ((32768, 32, 4096), "<64x64x16, 4 waves, 4 sets>"),            # N < 64: no direct loads
    # K of at most 16 slices and M >= 2048: several 64x64 tiles a CU
    ((4096, 4096, 256), "<64x64x16, 4 waves, 6 LDS stages>"),
    ((4096, 4096, 128), "<64x64x16, 4 waves>"),             # under 13 slices: register-staged
    ((4096, 4096, 512), "<256x128x16, 8 waves, 4 sets>"),
    ((1000, 4096, 256), "<128x128x16, 8 waves>"),
    # K <= 1024 and 256x128 tiles that leave a partial last wave: 64x64
    ((4608, 4608, 512), "<64x64x16, 4 waves, 6 LDS stages>"),    # 648 tiles, 2.53 a CU
    ((6144, 6144, 1024), "<64x64x16, 4 waves, 6 LDS stages>"),   # 1152 tiles, 4.5 a CU
    ((6144, 6144, 2048), "<256x128x16, 8 waves, 4 sets>"),       # longer K: split in parts
    ((8192, 6144, 512), "<256x128x16, 8 waves, 4 sets>"),        # 1536 tiles, 6 a CU
    # exactly three 128x128 tiles a CU, K >= 2048
    ((2048, 6144, 4096), "<128x128x16, 8 waves>"),
    ((2048, 6144, 1024), "<64x64x16, 4 waves, 6 LDS stages>"),
    # the larger tiles where they waste no more of the edges
    ((65536, 128, 2048), "<256x128x16, 8 waves, 4 sets>"),
    ((32768, 128, 4096), "<128x128x16, 8 waves>"),
    ((4000, 4200, 1027), "<256x128x16, 8 waves, 4 sets>"),
])
def test_auto_tile_class(shape, tile):
    d = tra.tra_gemm_describe(tra.AUTO, *shape)
    assert f"kernel=gemm_mfma_f32{tile} " in d, d


def _plan(variant, M, N, K):
    d = tra.tra_gemm_describe(variant, M, N, K)
    f = dict(kv.split("=", 1) for kv in d.split() if "=" in kv and not kv.startswith("kernel"))
    bm, bn, bk = map(int, f["tile"].split("x"))
    return (bm, bn, bk, int(f["grid"]), int(f["block"]), int(f["stream_k_tiles"]),
            int(f["stream_k_wgs"]), f["split"], int(f["workspace_bytes"]))


def test_split_plans_hold_their_invariants():
    # over seeded random shapes, the split planned for MI355X's 256 CUs
    # (planned at 4, 3 and 1 workgroups a CU for parts, 3 and 1 for runs)
    # keeps the shape of each form: the grid, the workgroups and the
    # workspace follow from the tile count, and parts cut each split tile
    # into 2..8 runs of at least 2 slices
    rng = np.random.default_rng(8)
    seen = set()
    for _ in range(400):
        M, N = (int(x) for x in rng.integers(1, 6000, 2))
        K = int(rng.choice([rng.integers(1, 64), rng.integers(64, 3000), rng.integers(3000, 20000)]))
        bm, bn, bk, grid, block, sk, wgs, form, ws = _plan(tra.MFMA_STREAMK, M, N, K)
        tiles = -(-M // bm) * -(-N // bn)
        ipt = -(-K // bk)
        seen.add(form)
        if form == "none":
            assert sk == 0 and wgs == 0 and ws == 0 and grid == tiles
        elif form == "parts":
            parts = wgs // sk
            assert wgs == sk * parts and 2 <= parts <= 8 and 2 * parts <= ipt
            # the deep 64 x 64 tile (4 register sets; a split launch stages
            # through registers) is planned at three workgroups a CU
            deep = "4 sets" in tra.tra_gemm_describe(tra.MFMA_STREAMK, M, N, K)
            wave = 256 * (1 if block == 512 else (3 if deep else 4))
            assert sk == tiles % wave and wgs <= wave
            assert grid == tiles + sk * (parts - 1) and ws == wgs * bm * bn * 4
        else:
            assert form == "runs" and 0 < sk <= tiles and 0 < wgs <= 256 * (1 if block == 512 else 3)
            assert grid == tiles + sk * (bm * bn // 4 // block - 1) and ws == 2 * wgs * bm * bn * 4
        # the unsplit rung never splits, and AUTO runs one of the two
        assert "split=none" in tra.tra_gemm_describe(tra.MFMA, M, N, K)
        auto = tra.tra_gemm_describe(tra.AUTO, M, N, K)
        assert "rung=mfma " in auto or f"split={form} " in auto
    assert seen == {"none", "parts", "runs"}


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no CPU fallback: with the library absent, every call raises before it
    # does anything
    monkeypatch.setattr(tra, "LIB_PATH", str(tmp_path / "libtra_gemm.so"))
    monkeypatch.setattr(tra, "_lib", None)
    calls = (lambda: tra.load(),
             lambda: tra.gemm_f32(4, 4, 4, 0, 4, 0, 4, 0, 4),
             lambda: tra.gemm_f32_variant(tra.MFMA, 4, 4, 4, 0, 4, 0, 4, 0, 4),
             lambda: tra.tra_gemm_describe(tra.AUTO, 4, 4, 4),
             lambda: tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, 4, 4, 4))
    for call in calls:
        with pytest.raises(RuntimeError, match="is not built"):
            call()
    assert tra._lib is None
