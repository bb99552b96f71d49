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


# --- the chart ------------------------------------------------------------------

def _svg_parts(svg):
    import xml.dom.minidom
    doc = xml.dom.minidom.parseString(svg)
    lines = [[tuple(map(float, p.split(","))) for p in pl.getAttribute("points").split()]
             for pl in doc.getElementsByTagName("polyline")]
    circles = [(float(c.getAttribute("cx")), float(c.getAttribute("cy")))
               for c in doc.getElementsByTagName("circle") if c.getElementsByTagName("title")]
    return lines, circles


def _on_polyline(pt, poly, tol=0.6):
    # both axes are logarithmic, so a roof is straight between its vertices
    x, y = pt
    for (xa, ya), (xb, yb) in zip(poly, poly[1:]):
        if min(xa, xb) - tol <= x <= max(xa, xb) + tol and xb != xa:
            if abs(ya + (yb - ya) * (x - xa) / (xb - xa) - y) <= tol:
                return True
    return False


def test_chart_points_on_and_under_the_roof():
    roofs = [{"label": "r", "peak_tflops": 100.0, "bw_tbps": 4.0}]   # ridge at 25 flop/B
    pts = [{"label": "on slope", "ai": 5.0, "tflops": 20.0, "series": "a"},
           {"label": "on flat", "ai": 400.0, "tflops": 100.0, "series": "a"},
           {"label": "at ridge", "ai": 25.0, "tflops": 100.0, "series": "b"},
           {"label": "below", "ai": 400.0, "tflops": 10.0, "series": "b"}]
    lines, circles = _svg_parts(rl.roofline_svg(pts, roofs, "t"))
    assert len(lines) == 1 and len(circles) == 4
    roof = lines[0]
    assert _on_polyline(circles[0], roof) and _on_polyline(circles[1], roof)
    assert _on_polyline(circles[2], roof)
    assert not _on_polyline(circles[3], roof)
    # SVG y grows downwards: the point below the roof has the larger y
    assert circles[3][1] > circles[1][1]
    # the kink of the roof is the ridge point
    assert any(abs(v[0] - circles[2][0]) < 0.6 and abs(v[1] - circles[2][1]) < 0.6 for v in roof)


def test_points_table_fractions():
    roofs = [{"label": "ds", "peak_tflops": 100.0, "bw_tbps": 4.0},
             {"label": "m", "peak_tflops": 80.0, "bw_tbps": 2.0, "unit": "mfma"}]
    pts = [{"label": "p", "ai": 10.0, "tflops": 20.0, "series": "s", "unit": "mfma"},
           {"label": "q", "ai": 1000.0, "tflops": 50.0, "series": "s", "unit": "valu"}]
    t = rl.points_table(pts, roofs).splitlines()
    # p: datasheet roof 4 x 10 = 40 (50%), own roof 2 x 10 = 20 (100%)
    assert t[2].split("|")[5:9] == [" 40 ", " 50.0 ", " 20 ", " 100.0 "]
    # q: datasheet roof 100 (50%); no measured roof for its unit
    assert t[3].split("|")[5:9] == [" 100 ", " 50.0 ", " – ", " – "]


def test_chart_from_bench_line():
    line = {"ladder": {"uniform1024": {"naive": {"tflops": 5.0, "unit": "valu"},
                                       "mfma": {"tflops": 90.0, "unit": "mfma"}}},
            "detail": {"measured_roofs": {"hbm_copy_tbps": 5.5, "mfma_fp32_tflops": 155.0,
                                          "valu_fp32_tflops": 102.5}}}
    traffic = {("mfma", "uniform1024"): 2 * rl.gemm_bytes(1024, 1024, 1024)}
    pts, roofs = rl.chart_from_bench(line, traffic)
    assert [r["peak_tflops"] for r in roofs] == [157.3, 155.0, 102.5]
    assert len(pts) == 3
    measured = [p for p in pts if "measured" in p["series"]]
    assert len(measured) == 1 and measured[0]["ai"] == pytest.approx(1024 / 12)
