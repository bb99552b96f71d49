"""Roofline arithmetic for the FP32 GEMM (host-side measurement helpers).

Definitions (page "Roofline & Tiling notes",
legato-user-group.github.io/tensor2silicon-lab/week04/researchers/jaehyeong):
  * arithmetic intensity AI = total flops / bytes the algorithm must move
    between HBM and the chip (section 1 "Arithmetic Intensity");
  * attainable performance = min(peak flops, bandwidth x AI) and the ridge
    (critical AI) = peak / bandwidth (the week's key points and section 2
    "Roofline");
  * a GEMM of N x N binary32 matrices reads A and B once and writes C once,
    12 N^2 bytes, for 2 N^3 flops, so AI = N / 6 (42.67 at N = 256); a vector
    add moves 12 N bytes for N flops, AI = 1/12 (section 1, worked examples).
Flop count 2*M*N*K (M*N*K multiplies and as many adds): page "GEMM kernel
test code & optimization (1024^3 experiment)", section "Mathematical
definition" (2.147e9 at 1024^3).

MI355X figures (AMD's public specification, not the pages): 256 CUs at up
to 2.4 GHz; dense FP32 157.3 TFLOP/s for both matrix (MFMA) and packed
vector instructions; HBM3E 8 TB/s.  The library's probes measure the roofs
actually reachable on the device (HBM copy bandwidth, FP32 MFMA and FP32
VALU rates; see tra_probe_* in include/tra_gemm.h).
"""
from __future__ import annotations

MI355X_CUS = 256
MI355X_CLOCK_GHZ = 2.4
# Dense FP32 peak, MFMA and packed VALU: 256 CU x 2.4 GHz x 256 flop/clk/CU.
PEAK_FP32_MFMA_TFLOPS = 157.3
HBM_TBPS = 8.0
ELEM_BYTES = 4


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def gemm_bytes(M: int, N: int, K: int, elem: int = ELEM_BYTES) -> int:
    """Compulsory HBM traffic: read A (M x K) and B (K x N), write C (M x N)."""
    return elem * (M * K + K * N + M * N)


def gemm_ai(M: int, N: int, K: int) -> float:
    return gemm_flops(M, N, K) / gemm_bytes(M, N, K)


def vector_add_ai(n: int) -> float:
    """n additions over 3 arrays of n binary32 values (two reads, one write)."""
    return n / (3 * ELEM_BYTES * n)


def ridge(peak_tflops: float = PEAK_FP32_MFMA_TFLOPS, bw_tbps: float = HBM_TBPS) -> float:
    """Critical AI in flop/byte where the two roofs meet."""
    return peak_tflops / bw_tbps


def roof_tflops(ai: float, peak_tflops: float = PEAK_FP32_MFMA_TFLOPS,
                bw_tbps: float = HBM_TBPS) -> float:
    """Attainable TFLOP/s at intensity ``ai``: min(peak, bandwidth x AI)."""
    return min(peak_tflops, bw_tbps * ai)


def bound(ai: float, peak_tflops: float = PEAK_FP32_MFMA_TFLOPS,
          bw_tbps: float = HBM_TBPS) -> str:
    return "hbm" if ai < ridge(peak_tflops, bw_tbps) else "compute"


def gemm_roofline(M: int, N: int, K: int, seconds: float,
                  peak_tflops: float = PEAK_FP32_MFMA_TFLOPS,
                  bw_tbps: float = HBM_TBPS) -> dict:
    """Achieved TFLOP/s of one GEMM taking ``seconds`` against its roofs."""
    fl = gemm_flops(M, N, K)
    by = gemm_bytes(M, N, K)
    ai = fl / by
    tflops = fl / seconds / 1e12
    roof = roof_tflops(ai, peak_tflops, bw_tbps)
    hbm_floor_s = by / (bw_tbps * 1e12)
    return {
        "flops": fl, "bytes": by, "ai": ai, "tflops": tflops, "roof_tflops": roof,
        "frac_of_roof": tflops / roof, "bound": bound(ai, peak_tflops, bw_tbps),
        "hbm_floor_s": hbm_floor_s, "frac_of_hbm_floor": hbm_floor_s / seconds,
        "achieved_gbps": by / seconds / 1e9,
    }
