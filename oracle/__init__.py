"""CPU oracle for single-precision GEMM, C = A x B (row-major).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports it and shares no code with
it.

The arithmetic lives in ``oracle_gemm.c`` (plain C, binary64 accumulation,
k summed in increasing order); this module only builds that file with gcc and
marshals numpy arrays into it.  What is computed, per element:

    C64[i, j] = sum_{k<K} A[i, k] * B[k, j]   (binary64, k ascending)
    C32[i, j] = C64[i, j] rounded once to binary32 (nearest even)
    S64[i, j] = sum_{k<K} |A[i, k] * B[k, j]|  (tolerance scale)

following the per-element definition of page "GEMM kernel test code &
optimization (1024^3 experiment)" (teach-meaning.tistory.com/1513), section
"Mathematical definition", in the order of the CPU triple loop of page
"[AutoMine++] #2 matmul trial and error" (velog.io/@levelstage/AutoMinepp2),
section "Intuitive implementation (by CPU)".

Parity status: pinned (see tests/test_oracle_pins.py); nothing is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")

_lib = None


def build() -> str:
    """Compile oracle_gemm.c into liboracle_gemm.so with gcc (always rebuilds)."""
    cmd = [
        "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
        "-pthread", "-std=c11", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, p, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, i64, c_int]
    lib.oracle_gemm.restype = c_int
    lib.oracle_gemm_entries.argtypes = [i64, i64, i64, p, i64, p, i64, i64, p, p,
                                        p, p, p, c_int]
    lib.oracle_gemm_entries.restype = c_int
    _lib = lib
    return lib


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _as_f32_2d(x: np.ndarray, name: str) -> np.ndarray:
    if not isinstance(x, np.ndarray) or x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 numpy array")
    if x.size and (x.strides[1] != 4 or x.strides[0] % 4 != 0 or x.strides[0] < 4 * x.shape[1]):
        raise ValueError(f"{name} must be row-major with unit column stride")
    return x


def _ld(x: np.ndarray) -> int:
    """Leading dimension (row pitch in elements) of a row-major view."""
    if x.size == 0 or x.shape[0] == 1:
        return max(1, x.shape[1])
    return x.strides[0] // 4


def _ptr(x: np.ndarray | None):
    return None if x is None else x.ctypes.data


@dataclass
class OracleResult:
    c64: np.ndarray   # float64 (M, N): the exact-order binary64 sum
    c32: np.ndarray   # float32 (M, N): c64 rounded once to binary32
    s64: np.ndarray   # float64 (M, N): sum of |products|


def gemm(A: np.ndarray, B: np.ndarray, K: int | None = None,
         nthreads: int | None = None) -> OracleResult:
    """Full C = A @ B of row-major float32 A (M x >=K) and B (>=K x N).

    ``A`` and ``B`` may be views with padded rows (leading dimension taken
    from the row stride).  ``K`` defaults to A's column count.
    """
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    M = A.shape[0]
    K = A.shape[1] if K is None else int(K)
    N = B.shape[1]
    if B.shape[0] < K or A.shape[1] < K:
        raise ValueError("inner dimensions do not match")
    lda = _ld(A)
    ldb = _ld(B)
    c64 = np.empty((M, N), np.float64)
    c32 = np.empty((M, N), np.float32)
    s64 = np.empty((M, N), np.float64)
    rc = _load().oracle_gemm(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(c64), _ptr(c32),
                             _ptr(s64), N, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm rejected its arguments (rc={rc})")
    return OracleResult(c64, c32, s64)


def gemm_entries(A: np.ndarray, B: np.ndarray, rows, cols, K: int | None = None,
                 nthreads: int | None = None) -> OracleResult:
    """Selected entries C[rows[e], cols[e]]; results are 1-D arrays of length e."""
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    M = A.shape[0]
    K = A.shape[1] if K is None else int(K)
    N = B.shape[1]
    if B.shape[0] < K or A.shape[1] < K:
        raise ValueError("inner dimensions do not match")
    rows = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int64).ravel()
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same length")
    n = rows.size
    c64 = np.empty(n, np.float64)
    c32 = np.empty(n, np.float32)
    s64 = np.empty(n, np.float64)
    rc = _load().oracle_gemm_entries(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), n,
                                     _ptr(rows), _ptr(cols),
                                     _ptr(c64), _ptr(c32), _ptr(s64),
                                     nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_gemm_entries rejected its arguments (rc={rc})")
    return OracleResult(c64, c32, s64)
