"""Seeded synthetic inputs for the FP32 GEMM workloads.

This module only makes input matrices; it holds none of the GEMM arithmetic.
It is the one piece shared by the CPU oracle's tests and the GPU path's tests
and benchmark, so both sides see identical bits.

Patterns:
  * integer patterns over the logical flat index, as in the host set-up of
    page "GEMM kernel test code & optimization (1024^3 experiment)"
    (teach-meaning.tistory.com/1513), section "Host code and timing":
    A[i, k] = ((i*K + k) mod 13) - 6 and B[k, j] = ((k*N + j) mod 7) - 3.
    The index is the logical one (i*K + k, k*N + j) whatever the leading
    dimension of the buffer is.
  * constants A = 0.5, B = 0.4, as in the CPU benchmark of page
    "[AutoMine++] #2 matmul trial and error" (velog.io/@levelstage/AutoMinepp2),
    section "Intuitive implementation (by CPU)".
  * seeded uniform[-1, 1) and normal(0, 1) in float32 from a torch CPU
    generator (the pages use no random data; A takes seed s, B seed s + 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def int_pattern_a(M: int, K: int) -> np.ndarray:
    """A[i, k] = ((i*K + k) mod 13) - 6 as float32, shape (M, K)."""
    row = (np.arange(M, dtype=np.int64) * K) % 13
    col = np.arange(K, dtype=np.int64) % 13
    out = np.empty((M, K), np.float32)
    step = max(1, (1 << 24) // max(K, 1))
    for r0 in range(0, M, step):
        r1 = min(M, r0 + step)
        out[r0:r1] = ((row[r0:r1, None] + col[None, :]) % 13 - 6).astype(np.float32)
    return out


def int_pattern_b(K: int, N: int) -> np.ndarray:
    """B[k, j] = ((k*N + j) mod 7) - 3 as float32, shape (K, N)."""
    row = (np.arange(K, dtype=np.int64) * N) % 7
    col = np.arange(N, dtype=np.int64) % 7
    out = np.empty((K, N), np.float32)
    step = max(1, (1 << 24) // max(N, 1))
    for r0 in range(0, K, step):
        r1 = min(K, r0 + step)
        out[r0:r1] = ((row[r0:r1, None] + col[None, :]) % 7 - 3).astype(np.float32)
    return out


def constant(rows: int, cols: int, value: float) -> np.ndarray:
    return np.full((rows, cols), np.float32(value), np.float32)


def uniform(rows: int, cols: int, seed: int) -> np.ndarray:
    """float32 uniform[-1, 1) from torch's CPU generator seeded with ``seed``."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    t = torch.empty((rows, cols), dtype=torch.float32)
    t.uniform_(-1.0, 1.0, generator=g)
    return t.numpy()


def normal(rows: int, cols: int, seed: int) -> np.ndarray:
    """float32 normal(0, 1) from torch's CPU generator seeded with ``seed``."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    t = torch.empty((rows, cols), dtype=torch.float32)
    t.normal_(0.0, 1.0, generator=g)
    return t.numpy()


def small_ints(rows: int, cols: int, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """float32 integers in [lo, hi] (exact products and sums for small K)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(rows, cols)).astype(np.float32)


def padded(x: np.ndarray, ld: int, fill: float = np.nan) -> np.ndarray:
    """Copy of row-major ``x`` in a buffer with leading dimension ``ld``.

    Returns the (rows, cols) view; the padding columns hold ``fill`` so a
    kernel that reads them shows up as a wrong (NaN) result.
    """
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("ld must be >= the column count")
    buf = np.full((rows, ld), np.float32(fill), np.float32)
    buf[:, :cols] = x
    return buf[:, :cols]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    kind: str          # "int", "const", "uniform", "normal"
    seed: int | None   # A uses seed, B uses seed + 1
    what: str

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def make(self) -> tuple[np.ndarray, np.ndarray]:
        M, N, K = self.M, self.N, self.K
        if self.kind == "int":
            return int_pattern_a(M, K), int_pattern_b(K, N)
        if self.kind == "const":
            return constant(M, K, 0.5), constant(K, N, 0.4)
        if self.kind == "uniform":
            return uniform(M, K, self.seed), uniform(K, N, self.seed + 1)
        if self.kind == "normal":
            return normal(M, K, self.seed), normal(K, N, self.seed + 1)
        raise ValueError(self.kind)


# The workloads: sizes, value distributions and seeds.
WORKLOADS = {
    w.name: w for w in [
        Workload("int256", 256, 256, 256, "int", None,
                 "256^3, integer patterns (exact results)"),
        Workload("const256", 256, 256, 256, "const", None,
                 "256^3, A=0.5, B=0.4 (C = 256*0.5*fl32(0.4))"),
        Workload("int1024", 1024, 1024, 1024, "int", None,
                 "1024^3, integer patterns (exact results)"),
        Workload("uniform1024", 1024, 1024, 1024, "uniform", 1024,
                 "1024^3, uniform[-1,1) seeds 1024/1025"),
        Workload("normal4096", 4096, 4096, 4096, "normal", 4096,
                 "4096^3, normal(0,1) seeds 4096/4097"),
        Workload("ragged", 3000, 2049, 1531, "uniform", 3000,
                 "3000x2049x1531, uniform[-1,1) seeds 3000/3001"),
        Workload("tall", 16384, 64, 16384, "uniform", 16384,
                 "16384x64x16384 tall-skinny, uniform[-1,1) seeds 16384/16385"),
        # One GPU's share when the two large shapes are split over 8 GPUs:
        # a slab of 512 rows of C (all of K and N), and a slab of 2048 of K.
        Workload("rowslab4096", 512, 4096, 4096, "normal", 4096,
                 "512x4096x4096 row slab (4096^3 over 8 GPUs), normal(0,1) seeds 4096/4097"),
        Workload("kslab_tall", 16384, 64, 2048, "uniform", 16384,
                 "16384x64x2048 K slab (tall-skinny over 8 GPUs), uniform[-1,1) seeds 16384/16385"),
    ]
}
