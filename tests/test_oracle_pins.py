"""Pins of the CPU oracle to facts other than itself.

Each pin is a function taking a GEMM callable ``f(A, B) -> OracleResult`` so
the same checks can be run against planted mistakes (see the mutant test at
the end): every plausible slip -- a dropped term, a wrong sign, a shifted
index, a transposed operand, binary32 accumulation -- must fail at least one
pin.

What the pins rest on:
  * closed form of the integer patterns (A = (i*K+k mod 13) - 6,
    B = (k*N+j mod 7) - 3, from the host set-up of page "GEMM kernel test code
    & optimization (1024^3 experiment)", section "Host code and timing"): the
    k sum is a sum over the residues k mod 91 weighted by their counts, a
    formula that never loops over k;
  * numpy's int64 matmul of the same integers (a library routine the oracle
    does not use);
  * the constant inputs 0.5 / 0.4 of page "[AutoMine++] #2 matmul trial and
    error", section "Intuitive implementation (by CPU)": C = K * 0.5 * fl32(0.4)
    exactly;
  * math.fsum (correctly rounded) on tiny shapes, with the textbook bound for
    recursive summation, and exact equality on small integers;
  * Freivalds' check and numpy's float64 matmul at 1024^3;
  * identities: A = I gives B; (AB)^T = B^T A^T bit for bit; K = 0 gives 0.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from tiling_roofline_analysis_amd import inputs

U = 2.0 ** -53  # unit roundoff of binary64


# ----------------------------------------------------------------------------
# independent references
# ----------------------------------------------------------------------------

def int_pattern_block(M: int, N: int, K: int) -> np.ndarray:
    """13 x 7 table T with C[i, j] = T[i mod 13, j mod 7] for the integer
    patterns, from residue counting (pure Python integers, no k loop)."""
    T = np.zeros((13, 7), np.int64)
    counts = [max(0, (K - 1 - c) // 91 + 1) for c in range(91)]
    for ir in range(13):
        for jr in range(7):
            tot = 0
            for c in range(91):
                if counts[c] == 0:
                    continue
                a = (ir * K + c) % 13 - 6
                b = (c * N + jr) % 7 - 3
                tot += counts[c] * a * b
            T[ir, jr] = tot
    return T


def int_pattern_expected(M: int, N: int, K: int, rows=None, cols=None) -> np.ndarray:
    T = int_pattern_block(M, N, K)
    if rows is None:
        rows = np.arange(M)
        cols = np.arange(N)
        return T[rows[:, None] % 13, cols[None, :] % 7]
    return T[np.asarray(rows) % 13, np.asarray(cols) % 7]


def tiny_cases():
    out = []
    for M in (1, 2, 3, 5):
        for N in (1, 2, 4, 7):
            for K in (1, 2, 3, 6, 8):
                out.append((M, N, K))
    for K in (15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129):
        out.append((3, 5, K))
    return out


# ----------------------------------------------------------------------------
# pins: each returns (ok, message)
# ----------------------------------------------------------------------------

def pin_int_closed_form(f, M=29, N=23, K=205):
    A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    r = f(A, B)
    exp = int_pattern_expected(M, N, K)
    ok = np.array_equal(r.c64, exp.astype(np.float64)) and np.array_equal(
        r.c32, exp.astype(np.float32))
    return ok, "integer-pattern closed form"


def pin_int_numpy(f, M=37, N=41, K=97):
    A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    r = f(A, B)
    exp = A.astype(np.int64) @ B.astype(np.int64)
    return np.array_equal(r.c64, exp.astype(np.float64)), "int64 numpy matmul"


def pin_constant(f, M=8, N=9, K=256):
    A, B = inputs.constant(M, K, 0.5), inputs.constant(K, N, 0.4)
    r = f(A, B)
    exact = K * 0.5 * float(np.float32(0.4))
    ok = bool(np.all(r.c64 == exact)) and bool(np.all(r.c32 == np.float32(exact)))
    return ok, "constant 0.5 x 0.4"


def pin_fsum(f, seed=7):
    rng = np.random.default_rng(seed)
    for (M, N, K) in tiny_cases():
        A = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        r = f(A, B)
        for i in range(M):
            for j in range(N):
                prods = [float(A[i, k]) * float(B[k, j]) for k in range(K)]
                ref = math.fsum(prods)
                mag = math.fsum(abs(p) for p in prods)
                bound = K * U * mag * 1.0001
                if not abs(r.c64[i, j] - ref) <= bound:
                    return False, f"fsum bound at {(M, N, K)} [{i},{j}]"
                if not abs(r.s64[i, j] - mag) <= bound:
                    return False, f"|product| sum at {(M, N, K)} [{i},{j}]"
        Ai = inputs.small_ints(M, K, seed + K)
        Bi = inputs.small_ints(K, N, seed + K + 1)
        ri = f(Ai, Bi)
        for i in range(M):
            for j in range(N):
                ref = sum(int(Ai[i, k]) * int(Bi[k, j]) for k in range(K))
                if ri.c64[i, j] != ref:
                    return False, f"small-integer exactness at {(M, N, K)}"
    return True, "fsum brute force"


def pin_identity(f):
    rng = np.random.default_rng(11)
    Bm = rng.standard_normal((19, 13)).astype(np.float32)
    eye = np.eye(19, dtype=np.float32)
    r = f(eye, Bm)
    ok1 = np.array_equal(r.c64, Bm.astype(np.float64))
    Am = rng.standard_normal((7, 19)).astype(np.float32)
    r2 = f(Am, eye)
    ok2 = np.array_equal(r2.c64, Am.astype(np.float64))
    return ok1 and ok2, "identity"


def pin_transpose(f):
    rng = np.random.default_rng(12)
    A = rng.uniform(-1, 1, (17, 33)).astype(np.float32)
    B = rng.uniform(-1, 1, (33, 9)).astype(np.float32)
    r = f(A, B)
    rt = f(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    return np.array_equal(r.c64, rt.c64.T), "(AB)^T = B^T A^T"


def pin_numpy_f64(f, M=48, N=40, K=300, seed=5):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    r = f(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    mag = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    ok = bool(np.all(np.abs(r.c64 - ref) <= 2 * K * U * mag + 1e-300))
    return ok, "numpy float64 matmul"


PINS = [pin_int_closed_form, pin_int_numpy, pin_constant, pin_fsum, pin_identity,
        pin_transpose, pin_numpy_f64]


# ----------------------------------------------------------------------------
# the oracle passes every pin
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(oracle_mod, pin):
    ok, what = pin(oracle_mod.gemm)
    assert ok, what


def test_closed_form_matches_int64_numpy():
    # the two independent references agree with each other
    for (M, N, K) in [(13, 7, 91), (30, 20, 200), (64, 33, 1531)]:
        A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
        assert np.array_equal(int_pattern_expected(M, N, K),
                              A.astype(np.int64) @ B.astype(np.int64))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (1024, 1024, 1024)])
def test_int_patterns_full(oracle_mod, M, N, K):
    A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    r = oracle_mod.gemm(A, B)
    exp = int_pattern_expected(M, N, K)
    assert np.array_equal(r.c64, exp.astype(np.float64))
    assert np.array_equal(r.c32, exp.astype(np.float32))
    assert np.array_equal(r.c64, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))


@pytest.mark.parametrize("name", ["normal4096", "ragged", "tall"])
def test_int_patterns_entries_full_size(oracle_mod, name):
    # the large shapes with the integer patterns, on sampled entries
    w = inputs.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    A, B = inputs.int_pattern_a(M, K), inputs.int_pattern_b(K, N)
    rng = np.random.default_rng(1)
    rows = np.concatenate([[0, M - 1], rng.integers(0, M, 300)])
    cols = np.concatenate([[0, N - 1], rng.integers(0, N, 300)])
    r = oracle_mod.gemm_entries(A, B, rows, cols)
    exp = int_pattern_expected(M, N, K, rows, cols)
    assert np.array_equal(r.c64, exp.astype(np.float64))


def test_constant_256_exact_bits(oracle_mod):
    w = inputs.WORKLOADS["const256"]
    A, B = w.make()
    r = oracle_mod.gemm(A, B)
    assert np.all(r.c64 == 51.20000076293945)
    assert np.all(r.c32.view(np.uint32) == 0x424CCCCD)


def test_freivalds_1024_uniform(oracle_mod):
    A, B = inputs.WORKLOADS["uniform1024"].make()
    r = oracle_mod.gemm(A, B)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    rng = np.random.default_rng(3)
    for _ in range(3):
        x = rng.standard_normal(B.shape[1])
        lhs = r.c64 @ x
        rhs = A64 @ (B64 @ x)
        scale = r.s64 @ np.abs(x) + np.abs(A64) @ (np.abs(B64) @ np.abs(x))
        K = A.shape[1]
        assert np.all(np.abs(lhs - rhs) <= 4 * (K + B.shape[1]) * U * scale)
    # row sums: sum_j C_ij = sum_k A_ik (sum_j B_kj)
    rs = A64 @ B64.sum(axis=1)
    assert np.allclose(r.c64.sum(axis=1), rs, rtol=0, atol=1e-9 * r.s64.sum(axis=1).max())


def test_s64_is_abs_product(oracle_mod):
    rng = np.random.default_rng(9)
    A = rng.standard_normal((31, 77)).astype(np.float32)
    B = rng.standard_normal((77, 29)).astype(np.float32)
    r = oracle_mod.gemm(A, B)
    ref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(r.s64 - ref) <= 2 * 77 * U * ref)
    assert np.all(np.abs(r.c64) <= r.s64)


def test_c32_is_rounded_c64(oracle_mod):
    rng = np.random.default_rng(10)
    A = rng.standard_normal((20, 50)).astype(np.float32)
    B = rng.standard_normal((50, 30)).astype(np.float32)
    r = oracle_mod.gemm(A, B)
    assert np.array_equal(r.c32, r.c64.astype(np.float32))


def test_k_zero_and_empty(oracle_mod):
    A = np.zeros((4, 0), np.float32)
    B = np.zeros((0, 5), np.float32)
    r = oracle_mod.gemm(A, B)
    assert r.c64.shape == (4, 5) and np.all(r.c64 == 0) and np.all(r.c32 == 0)
    r = oracle_mod.gemm(np.zeros((0, 3), np.float32), np.zeros((3, 5), np.float32))
    assert r.c64.shape == (0, 5)


def test_entries_equal_full(oracle_mod):
    rng = np.random.default_rng(4)
    A = rng.uniform(-1, 1, (45, 123)).astype(np.float32)
    B = rng.uniform(-1, 1, (123, 51)).astype(np.float32)
    full = oracle_mod.gemm(A, B)
    rows = rng.integers(0, 45, 200)
    cols = rng.integers(0, 51, 200)
    e = oracle_mod.gemm_entries(A, B, rows, cols)
    assert np.array_equal(e.c64, full.c64[rows, cols])
    assert np.array_equal(e.c32, full.c32[rows, cols])
    assert np.array_equal(e.s64, full.s64[rows, cols])


def test_thread_count_independent(oracle_mod):
    rng = np.random.default_rng(6)
    A = rng.standard_normal((33, 257)).astype(np.float32)
    B = rng.standard_normal((257, 19)).astype(np.float32)
    r1 = oracle_mod.gemm(A, B, nthreads=1)
    r7 = oracle_mod.gemm(A, B, nthreads=7)
    assert np.array_equal(r1.c64, r7.c64)


def test_padded_leading_dimensions(oracle_mod):
    rng = np.random.default_rng(8)
    A = rng.uniform(-1, 1, (21, 35)).astype(np.float32)
    B = rng.uniform(-1, 1, (35, 18)).astype(np.float32)
    ref = oracle_mod.gemm(A, B)
    Ap = inputs.padded(A, 40)   # padding holds NaN: reading it would show
    Bp = inputs.padded(B, 23)
    r = oracle_mod.gemm(Ap, Bp)
    assert np.array_equal(r.c64, ref.c64)


def test_invalid_arguments(oracle_mod):
    A = np.zeros((3, 4), np.float32)
    B = np.zeros((5, 2), np.float32)
    with pytest.raises(ValueError):
        oracle_mod.gemm(A, B, K=5)      # K larger than A's columns
    with pytest.raises(ValueError):
        oracle_mod.gemm_entries(np.zeros((3, 4), np.float32), np.zeros((4, 2), np.float32),
                                [3], [0])   # row out of range
    with pytest.raises(TypeError):
        oracle_mod.gemm(A.astype(np.float64), B)


# ----------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------

def _mutants(oracle_mod):
    g = oracle_mod.gemm

    def dropped_last_term(A, B):
        K = A.shape[1]
        if K <= 1:
            return g(A[:, :0] if K == 1 else A, B[:0] if K == 1 else B)
        return g(np.ascontiguousarray(A[:, :K - 1]), np.ascontiguousarray(B[:K - 1]))

    def dropped_first_term(A, B):
        return g(np.ascontiguousarray(A[:, 1:]), np.ascontiguousarray(B[1:]))

    def wrong_sign_odd_k(A, B):
        s = np.where(np.arange(A.shape[1]) % 2 == 1, -1.0, 1.0).astype(np.float32)
        return g(np.ascontiguousarray(A * s[None, :]), B)

    def shifted_row(A, B):
        return g(np.ascontiguousarray(np.roll(A, 1, axis=0)), B)

    def shifted_k_in_b(A, B):
        return g(A, np.ascontiguousarray(np.roll(B, 1, axis=0)))

    def transposed_b(A, B):
        K, N = B.shape
        Bt = np.ascontiguousarray(B.T.reshape(K, N))   # B read column-major
        return g(A, Bt)

    def transposed_a(A, B):
        M, K = A.shape
        At = np.ascontiguousarray(A.T.reshape(M, K))   # A read column-major
        return g(At, B)

    def float32_accumulation(A, B):
        r = g(A, B)
        M, K = A.shape
        N = B.shape[1]
        acc = np.zeros((M, N), np.float32)
        for k in range(K):
            acc = (acc + A[:, k:k + 1] * B[k:k + 1, :]).astype(np.float32)
        r.c64 = acc.astype(np.float64)
        r.c32 = acc
        return r

    return [dropped_last_term, dropped_first_term, wrong_sign_odd_k, shifted_row,
            shifted_k_in_b, transposed_b, transposed_a, float32_accumulation]


def test_pins_catch_planted_mistakes(oracle_mod):
    for mutant in _mutants(oracle_mod):
        failed = []
        for pin in PINS:
            try:
                ok, what = pin(mutant)
            except Exception:   # a crash also counts as caught
                ok, what = False, pin.__name__
            if not ok:
                failed.append(what)
        assert failed, f"no pin catches the planted mistake {mutant.__name__}"
