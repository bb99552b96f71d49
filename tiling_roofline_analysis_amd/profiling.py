"""Summaries of rocprofv3 results for the GEMM kernels (host-side tooling).

rocprofv3 (ROCm 7) writes its results as a SQLite database (rocpd format).
This module turns one into the short text summaries kept under profiles/:

  trace    per-kernel dispatch count and average / min / max duration from a
           `rocprofv3 --kernel-trace --stats` run;
  traffic  HBM bytes per launch of one GEMM kernel from two `--pmc` runs
           (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each
           scaled by what the same counter reads for a plain device copy of
           known size in the same run (`bench.py --copy-calibration`).

The traffic summary records a digest of the kernel sources; bench.py reports
the stored traffic only while that digest matches the current sources.

    python -m tiling_roofline_analysis_amd.profiling trace DB --cmd "..."
    python -m tiling_roofline_analysis_amd.profiling traffic FETCH_DB WRITE_DB \\
        --match "MfmaTile<64, 64" --grid 65536 --workload uniform1024 --cmd "..."
"""
from __future__ import annotations

import argparse
import hashlib
import re
import os
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")

# Bytes moved per launch by the calibration copy (bench.py --copy-calibration).
COPY_BYTES = 64 << 22    # 64 Mi floats = 256 MiB read and 256 MiB written
COPY_KERNEL = "copyBuffer"


def _code_only(text: str) -> str:
    """C++ source with comments and blank space removed (string literals
    with comment markers do not occur in these files)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files=("gemm_mfma.hip", "gemm_internal.h")) -> str:
    """Short sha256 of the code (comments and spacing aside) of the MFMA
    rung's HIP sources: a counter reading is current while this matches."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(HERE, "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_gemm_mfma_f32_{workload}.txt")


def stored_traffic(workload: str):
    """HBM bytes per launch from profiles/, or None if absent or stale."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _db(path):
    return sqlite3.connect(f"file:{path}?mode=ro", uri=True)


def trace_summary(db: str, cmd: str) -> str:
    c = _db(db)
    rows = c.execute(
        "select name, grid_x*grid_y*grid_z, workgroup_x*workgroup_y*workgroup_z, count(*), "
        "avg(duration), min(duration), max(duration), sum(duration) from kernels "
        "group by name, grid_x, grid_y, grid_z order by sum(duration) desc").fetchall()
    out = [f"# rocprofv3 kernel trace summary", "",
           f"command: `{cmd}`", "",
           "| kernel | grid (lanes) | block | dispatches | avg us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for name, grid, wg, n, avg, mn, mx, _ in rows:
        short = name.replace("(anonymous namespace)::", "").split("(long")[0]
        out.append(f"| `{short}` | {grid} | {wg} | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                   f"{mx / 1e3:.2f} |")
    return "\n".join(out) + "\n"


def _counter(db, match, grid):
    c = _db(db)
    rows = c.execute(
        "select kernel_name, grid_size, counter_name, avg(value), count(*) from counters_collection "
        "group by kernel_name, grid_size, counter_name").fetchall()
    copy = [r for r in rows if COPY_KERNEL in r[0]]
    gemm = [r for r in rows if match in r[0] and (grid is None or r[1] == grid)]
    if not copy or len(gemm) != 1:
        raise SystemExit(f"{db}: expected one calibration copy and one GEMM kernel "
                         f"(found {len(copy)} / {len(gemm)})")
    big = max(copy, key=lambda r: r[1])
    return gemm[0], big


def traffic_summary(fetch_db, write_db, match, grid, workload, cmd, algorithmic_bytes):
    g_f, c_f = _counter(fetch_db, match, grid)
    g_w, c_w = _counter(write_db, match, grid)
    fetch_scale = COPY_BYTES / (c_f[3] * 1024.0)
    write_scale = COPY_BYTES / (c_w[3] * 1024.0)
    read_b = g_f[3] * 1024.0 * fetch_scale
    write_b = g_w[3] * 1024.0 * write_scale
    total = read_b + write_b
    lines = [
        f"# HBM traffic of one GEMM launch from rocprofv3 counters",
        f"# FETCH_SIZE pass: {cmd.format(counter='FETCH_SIZE')}",
        f"# WRITE_SIZE pass: {cmd.format(counter='WRITE_SIZE')}",
        f"# kernel: {g_f[0].replace('(anonymous namespace)::', '').split('(long')[0]}",
        f"# calibration: plain device copy of {COPY_BYTES} bytes ({c_f[0]}):",
        f"#   FETCH_SIZE reads {c_f[3]:.1f} KiB -> scale {fetch_scale:.4f};"
        f" WRITE_SIZE reads {c_w[3]:.1f} KiB -> scale {write_scale:.4f}",
        f"workload = {workload}",
        f"grid_lanes = {g_f[1]}",
        f"dispatches = {g_f[4]}",
        f"fetch_size_kib = {g_f[3]:.1f}",
        f"write_size_kib = {g_w[3]:.1f}",
        f"fetch_scale = {fetch_scale:.4f}",
        f"write_scale = {write_scale:.4f}",
        f"hbm_read_bytes_per_launch = {read_b:.0f}",
        f"hbm_write_bytes_per_launch = {write_b:.0f}",
        f"hbm_bytes_per_launch = {total:.0f}",
        f"algorithmic_bytes_per_launch = {algorithmic_bytes}",
        f"traffic_over_algorithmic = {total / algorithmic_bytes:.3f}",
        f"source_digest = {source_digest()}",
    ]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description="summarise rocprofv3 results")
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("fetch_db")
    f.add_argument("write_db")
    f.add_argument("--match", required=True)
    f.add_argument("--grid", type=int, default=None)
    f.add_argument("--workload", required=True)
    f.add_argument("--cmd", required=True, help="profiling command with {counter}")
    args = ap.parse_args(argv)
    if args.what == "trace":
        sys.stdout.write(trace_summary(args.db, args.cmd))
    else:
        sys.path.insert(0, ROOT)
        from tiling_roofline_analysis_amd import inputs, roofline
        w = inputs.WORKLOADS[args.workload]
        sys.stdout.write(traffic_summary(args.fetch_db, args.write_db, args.match, args.grid,
                                         args.workload, args.cmd,
                                         roofline.gemm_bytes(w.M, w.N, w.K)))


if __name__ == "__main__":
    main()
