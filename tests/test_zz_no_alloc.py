"""gemm_f32_variant_noalloc on the GPU: the entry point that allocates
nothing (its split's partial tiles live in a scratch array that is part of
the library) against gemm_f32_variant, whose split uses the library's
allocated workspace.  Both run the same kernels with a K-ordered reduction,
so results must be bitwise equal; they are also checked against the CPU
oracle (1e-5 * sum |A_ik B_kj| on random floats, exact on integers).  Two
calls in a row, the second smaller, so the second reads partial tiles over
whatever the first left in the shared array."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tiling_roofline_analysis_amd as tra
from tiling_roofline_analysis_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tra.load()


def dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def both(variant, M, N, K, A, B):
    """C from the no-alloc entry point and from gemm_f32_variant."""
    import torch
    h = torch.cuda.current_stream().cuda_stream
    out = []
    for call in (tra.gemm_f32_variant_noalloc, tra.gemm_f32_variant):
        C = torch.full((M, N), float("nan"), device="cuda:0")
        st = call(variant, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N, h)
        assert st == tra.TRA_OK, f"{call.__name__}: {tra.tra_status_string(st)}"
        out.append(C)
    torch.cuda.synchronize()
    return out


# (first, second) shapes: the second is smaller; the forms of the split
PAIRS = [
    ((3000, 2049, 1531), (300, 500, 203), "parts", "parts"),
    ((4000, 4200, 1027), (1500, 1500, 77), "parts", "runs"),
    ((1152, 1152, 8192), (257, 129, 1000), "runs", "parts"),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[2]}-{p[3]}")
def test_noalloc_matches_gemm_f32_variant_twice(pair):
    first, second, f1, f2 = pair
    assert first[0] * first[1] * first[2] > second[0] * second[1] * second[2]
    for (M, N, K), form, seed in ((first, f1, 11), (second, f2, 12)):
        d = tra.tra_gemm_describe(tra.MFMA_STREAMK, M, N, K)
        print(f"[case] noalloc split={form} {M}x{N}x{K} ({d})", flush=True)
        assert f"split={form} " in d
        need = tra.tra_gemm_workspace_size(tra.MFMA_STREAMK, M, N, K)
        assert 0 < need <= tra.STATIC_SCRATCH_BYTES
        A, B = inputs.uniform(M, K, seed), inputs.uniform(K, N, seed + 1)
        C0, C1 = both(tra.MFMA_STREAMK, M, N, K, dev(A), dev(B))
        assert np.isfinite(C0.cpu().numpy()).all()
        assert C0.equal(C1), f"{M}x{N}x{K}: no-alloc differs from gemm_f32_variant"
        rng = np.random.default_rng(M)
        rows = np.concatenate([rng.integers(0, M, 4000), np.arange(M), np.full(N, M - 1)])
        cols = np.concatenate([rng.integers(0, N, 4000), np.full(M, N - 1), np.arange(N)])
        ref = oracle.gemm_entries(A, B, rows, cols)
        err = np.abs(C0.cpu().numpy()[rows, cols].astype(np.float64) - ref.c64)
        assert np.all(err <= TOL * ref.s64)


def test_noalloc_auto_and_unsplit_rungs_on_integer_patterns():
    # AUTO and the rungs that need no scratch run through the same entry
    # point; integer patterns are exact
    M, N, K = 3000, 2049, 1531
    A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    ii, jj = np.meshgrid(np.arange(13), np.arange(7), indexing="ij")
    per = oracle.gemm_entries(A, B, ii.ravel(), jj.ravel()).c32.reshape(ii.shape)
    exp = per[np.arange(M)[:, None] % 13, np.arange(N)[None, :] % 7]
    dA, dB = dev(A), dev(B)
    for v in (tra.AUTO, tra.MFMA, tra.REGBLOCK_DB):
        C0, C1 = both(v, M, N, K, dA, dB)
        assert np.array_equal(C0.cpu().numpy(), exp), tra.tra_gemm_variant_name(v)
        assert C0.equal(C1)
