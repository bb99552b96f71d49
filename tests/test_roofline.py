"""Host-side roofline helpers against the numbers the pages print
(tests/golden/pages_values.json, each entry with its page and section)."""
import json
import os

import pytest

from tiling_roofline_analysis_amd import roofline as rl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def g(key):
    return GOLDEN[key]["value"]


def test_flops_1024_matches_page():
    fl = rl.gemm_flops(1024, 1024, 1024)
    assert fl == 2 * 1024 ** 3 == 2147483648
    assert float(f"{fl:.3e}") == g("gemm_flops_1024")


def test_page_gflops_from_times():
    fl = rl.gemm_flops(1024, 1024, 1024)
    # the page's GFLOP/s are its flop count over its times, to 3 digits
    assert round(fl / (g("naive_avg_ms_1024") * 1e-3) / 1e9) == g("naive_gflops_1024")
    assert round(fl / (g("tiled_avg_ms_1024") * 1e-3) / 1e9) == g("tiled_gflops_1024")
    assert round(g("tiled_avg_ms_1024") / g("naive_avg_ms_1024"), 4) == g("tiled_over_naive")


def test_matmul_ai_n256_matches_page():
    assert rl.gemm_bytes(256, 256, 256) == g("matmul_bytes_factor") * 256 ** 2
    assert rl.gemm_ai(256, 256, 256) == pytest.approx(256 / 6)
    assert round(rl.gemm_ai(256, 256, 256), 2) == g("ai_matmul_n256")


def test_vector_add_ai_matches_page():
    assert round(rl.vector_add_ai(1 << 20), 3) == g("ai_vector_add")


def test_roof_is_min_of_peak_and_bw_times_ai():
    r = rl.ridge()
    assert r == pytest.approx(157.3 / 8.0)
    assert rl.roof_tflops(r / 2) == pytest.approx(8.0 * r / 2)
    assert rl.roof_tflops(r * 2) == pytest.approx(157.3)
    assert rl.bound(r / 2) == "hbm" and rl.bound(r * 2) == "compute"


@pytest.mark.parametrize("M,N,K,ai", [
    (256, 256, 256, 42.67), (1024, 1024, 1024, 170.67), (4096, 4096, 4096, 682.67),
    (3000, 2049, 1531, 339.09), (16384, 64, 16384, 31.75)])
def test_config_intensities(M, N, K, ai):
    assert round(rl.gemm_ai(M, N, K), 2) == ai
    # every configured shape sits right of the ridge (compute-bound roof)
    assert rl.bound(rl.gemm_ai(M, N, K)) == "compute"


def test_fp32_peak_from_unit_counts():
    # 256 CUs x 2.4 GHz x 256 flop per clock per CU
    assert rl.MI355X_CUS * rl.MI355X_CLOCK_GHZ * 256 / 1e3 == pytest.approx(
        rl.PEAK_FP32_MFMA_TFLOPS, rel=1e-3)


def test_gemm_roofline_report():
    rep = rl.gemm_roofline(1024, 1024, 1024, 20e-6)
    assert rep["tflops"] == pytest.approx(2147483648 / 20e-6 / 1e12)
    assert rep["frac_of_roof"] == pytest.approx(rep["tflops"] / 157.3)
    assert rep["bound"] == "compute"
