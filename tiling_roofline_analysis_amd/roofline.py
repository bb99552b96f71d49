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


# --- the roofline chart -------------------------------------------------------
#
# The pages' deliverable is a roofline chart: log-log axes of arithmetic
# intensity (flop/byte) against performance, the roof min(peak, BW x AI),
# and each kernel drawn as an "achieved value" point under it (page "Roofline
# & Tiling notes", section 2 "Roofline" and the week's key points).  The
# chart here is plain SVG text, so it needs no plotting package.

def _log_scale(v: float, lo: float, hi: float, a: float, b: float) -> float:
    import math
    return a + (math.log10(v) - math.log10(lo)) / (math.log10(hi) - math.log10(lo)) * (b - a)


def roofline_svg(points, roofs, title: str, ai_range=(0.05, 2000.0),
                 tflops_range=(0.5, 400.0), width: int = 800, height: int = 540) -> str:
    """SVG roofline chart.

    points: dicts with "label", "ai" (flop/byte), "tflops" and "series"
            (points of one series share a colour);
    roofs:  dicts with "label", "peak_tflops", "bw_tbps", and optionally
            "dash" (True for a dashed line).
    Points outside the axis ranges are clamped to the frame.
    """
    import html
    ml, mr, mt, mb = 70, 200, 40, 55
    x0, x1, y0, y1 = ml, width - mr, height - mb, mt
    lo_x, hi_x = ai_range
    lo_y, hi_y = tflops_range

    def X(ai):
        return _log_scale(min(max(ai, lo_x), hi_x), lo_x, hi_x, x0, x1)

    def Y(tf):
        return _log_scale(min(max(tf, lo_y), hi_y), lo_y, hi_y, y0, y1)

    palette = ["#1f77b4", "#d62728", "#2ca02c", "#9467bd", "#ff7f0e", "#8c564b", "#e377c2"]
    out = [f'<svg xmlns="http://www.w3.org/2000/svg" width="{width}" height="{height}" '
           f'font-family="sans-serif" font-size="11">',
           f'<rect x="0" y="0" width="{width}" height="{height}" fill="white"/>',
           f'<text x="{width / 2:.0f}" y="20" text-anchor="middle" font-size="14">'
           f'{html.escape(title)}</text>',
           f'<rect x="{x0}" y="{y1}" width="{x1 - x0}" height="{y0 - y1}" fill="none" '
           f'stroke="black"/>']
    # decade grid and tick labels
    import math
    for e in range(math.ceil(math.log10(lo_x)), math.floor(math.log10(hi_x)) + 1):
        x = X(10.0 ** e)
        out.append(f'<line x1="{x:.1f}" y1="{y0}" x2="{x:.1f}" y2="{y1}" stroke="#ddd"/>')
        out.append(f'<text x="{x:.1f}" y="{y0 + 15}" text-anchor="middle">{10.0 ** e:g}</text>')
    for e in range(math.ceil(math.log10(lo_y)), math.floor(math.log10(hi_y)) + 1):
        y = Y(10.0 ** e)
        out.append(f'<line x1="{x0}" y1="{y:.1f}" x2="{x1}" y2="{y:.1f}" stroke="#ddd"/>')
        out.append(f'<text x="{x0 - 6}" y="{y + 4:.1f}" text-anchor="end">{10.0 ** e:g}</text>')
    out.append(f'<text x="{(x0 + x1) / 2:.0f}" y="{height - 15}" text-anchor="middle">'
               f'arithmetic intensity (flop/byte)</text>')
    out.append(f'<text x="18" y="{(y0 + y1) / 2:.0f}" text-anchor="middle" '
               f'transform="rotate(-90 18 {(y0 + y1) / 2:.0f})">TFLOP/s</text>')
    # roofs: the sloped part BW x AI up to the ridge, then flat at the peak
    ly = y1 + 10
    for r in roofs:
        ridge_ai = r["peak_tflops"] / r["bw_tbps"]
        a_lo = max(lo_x, lo_y / r["bw_tbps"])
        pts = [(a_lo, r["bw_tbps"] * a_lo), (ridge_ai, r["peak_tflops"]), (hi_x, r["peak_tflops"])]
        path = " ".join(f"{X(a):.1f},{Y(t):.1f}" for a, t in pts)
        dash = ' stroke-dasharray="6,4"' if r.get("dash") else ""
        out.append(f'<polyline points="{path}" fill="none" stroke="black" stroke-width="1.5"{dash}/>')
        out.append(f'<line x1="{x1 + 10}" y1="{ly}" x2="{x1 + 30}" y2="{ly}" stroke="black"'
                   f' stroke-width="1.5"{dash}/>')
        out.append(f'<text x="{x1 + 35}" y="{ly + 4}">{html.escape(r["label"])}</text>')
        ly += 16
    # points, one colour per series
    series = []
    for p in points:
        if p["series"] not in series:
            series.append(p["series"])
    ly += 8
    for i, s in enumerate(series):
        c = palette[i % len(palette)]
        out.append(f'<circle cx="{x1 + 20}" cy="{ly}" r="4" fill="{c}"/>')
        out.append(f'<text x="{x1 + 35}" y="{ly + 4}">{html.escape(s)}</text>')
        ly += 16
    for p in points:
        c = palette[series.index(p["series"]) % len(palette)]
        x, y = X(p["ai"]), Y(p["tflops"])
        out.append(f'<circle cx="{x:.1f}" cy="{y:.1f}" r="4" fill="{c}">'
                   f'<title>{html.escape(p["label"])}: AI {p["ai"]:.3g}, '
                   f'{p["tflops"]:.3g} TFLOP/s</title></circle>')
        out.append(f'<text x="{x + 6:.1f}" y="{y - 5:.1f}" font-size="9">'
                   f'{html.escape(p["label"])}</text>')
    out.append("</svg>")
    return "\n".join(out) + "\n"


def points_table(points, roofs) -> str:
    """Markdown table of the chart's points, each against the datasheet roof
    (the first of `roofs`) and against the measured roof of the unit it runs
    on (the roof whose "unit" matches the point's, if any)."""
    rows = ["| point | series | AI (flop/B) | TFLOP/s | datasheet roof at this AI | % of it "
            "| measured roof of its unit at this AI | % of it |",
            "|---|---|---|---|---|---|---|---|"]
    ds = roofs[0]
    for p in points:
        r0 = roof_tflops(p["ai"], ds["peak_tflops"], ds["bw_tbps"])
        own = [r for r in roofs[1:] if r.get("unit") and r["unit"] == p.get("unit")]
        if own:
            r1 = roof_tflops(p["ai"], own[0]["peak_tflops"], own[0]["bw_tbps"])
            m = f"{r1:.4g} | {100 * p['tflops'] / r1:.1f}"
        else:
            m = "– | –"
        rows.append(f"| {p['label']} | {p['series']} | {p['ai']:.4g} | {p['tflops']:.4g} | "
                    f"{r0:.4g} | {100 * p['tflops'] / r0:.1f} | {m} |")
    return "\n".join(rows) + "\n"


def chart_from_bench(line: dict, ladder_traffic: dict):
    """Points and roofs of the roofline chart from one bench.py JSON line:
    each rung at each timed shape, placed at the algorithmic intensity and,
    where counters were taken for the current sources (ladder_traffic:
    {(rung, workload): HBM bytes per launch}), at the intensity of its
    measured HBM traffic.  Roofs: the datasheet's, and the measured MFMA
    and VALU roofs with the measured copy bandwidth when present."""
    from tiling_roofline_analysis_amd import inputs
    points = []
    for wname, rungs in line.get("ladder", {}).items():
        w = inputs.WORKLOADS[wname]
        shape = f"{w.M}^3" if w.M == w.N == w.K else f"{w.M}x{w.N}x{w.K}"
        for rung, e in rungs.items():
            unit = e.get("unit")
            points.append({"label": f"{rung} {shape}", "ai": gemm_ai(w.M, w.N, w.K),
                           "tflops": e["tflops"], "unit": unit,
                           "series": "at algorithmic AI (A, B read once, C written once)"})
            hbm = ladder_traffic.get((rung, wname))
            if hbm:
                points.append({"label": f"{rung} {shape}",
                               "ai": gemm_flops(w.M, w.N, w.K) / hbm, "tflops": e["tflops"],
                               "unit": unit, "series": "at measured HBM traffic (rocprofv3)"})
    roofs = [{"label": f"datasheet {PEAK_FP32_MFMA_TFLOPS} TF, {HBM_TBPS} TB/s",
              "peak_tflops": PEAK_FP32_MFMA_TFLOPS, "bw_tbps": HBM_TBPS}]
    m = (line.get("detail") or {}).get("measured_roofs")
    if m:
        for unit, key in (("mfma", "mfma_fp32_tflops"), ("valu", "valu_fp32_tflops")):
            roofs.append({"label": f"measured {unit.upper()} {m[key]} TF, "
                                   f"{m['hbm_copy_tbps']} TB/s",
                          "peak_tflops": m[key], "bw_tbps": m["hbm_copy_tbps"], "dash": True,
                          "unit": unit})
    return points, roofs


def write_chart(line: dict, ladder_traffic: dict, svg_path=None, table_path=None):
    points, roofs = chart_from_bench(line, ladder_traffic)
    device = (line.get("detail") or {}).get("device", "one GPU")
    if svg_path:
        with open(svg_path, "w") as fh:
            fh.write(roofline_svg(points, roofs, f"FP32 GEMM ladder on {device}"))
    if table_path:
        with open(table_path, "w") as fh:
            fh.write(f"# Roofline points of the FP32 GEMM ladder on {device}\n\n")
            fh.write(points_table(points, roofs))


def main(argv=None):
    """python -m tiling_roofline_analysis_amd.roofline BENCH_JSON --svg F --table F"""
    import argparse
    import json
    import os
    import sys
    ap = argparse.ArgumentParser(description="roofline chart from a bench.py JSON line")
    ap.add_argument("bench_json")
    ap.add_argument("--svg")
    ap.add_argument("--table")
    args = ap.parse_args(argv)
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from tiling_roofline_analysis_amd.profiling import stored_ladder_traffic
    with open(args.bench_json) as fh:
        line = json.loads(fh.read().strip().splitlines()[-1])
    write_chart(line, stored_ladder_traffic(), args.svg, args.table)


if __name__ == "__main__":
    main()
