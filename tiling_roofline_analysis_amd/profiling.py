"""Summaries of rocprofv3 results for the GEMM kernels (host-side tooling).

rocprofv3 (ROCm 7) writes its results as a SQLite database (rocpd format).
This module turns one into the short text summaries kept under profiles/:

  trace    per-kernel dispatch count and average / min / max duration from a
           `rocprofv3 --kernel-trace --stats` run;
  traffic  HBM bytes per launch of one GEMM kernel from two `--pmc` runs
           (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each
           scaled by what the same counter reads for a plain device copy of
           known size in the same run (`bench.py --copy-calibration`);
  ladder   the same for every rung of the ladder at both configured shapes
           (bench.py run with its ladder), the points of the roofline chart;
  counters SQ instruction, LDS and MFMA counters of every rung from one
           `--pmc` pass over bench.py's ladder;
  drive    runs one configured workload through the C ABI (the library's
           own choice of kernels) a given number of times, after a plain
           device copy of known size: the program to profile, one workload
           per process, so that every GEMM kernel in its results belongs to
           that workload;
  configs  SQ counters of the kernels of each workload from such runs.

The traffic summary records a digest of the kernel sources; bench.py reports
the stored traffic only while that digest matches the current sources.

    python -m tiling_roofline_analysis_amd.profiling trace DB --cmd "..."
    python -m tiling_roofline_analysis_amd.profiling drive ragged --reps 20
    python -m tiling_roofline_analysis_amd.profiling traffic FETCH_DB WRITE_DB \\
        --workload ragged --cmd "..."
    python -m tiling_roofline_analysis_amd.profiling configs --cmd "..." ragged=DB ...
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


def _short(name):
    return name.replace("(anonymous namespace)::", "").split("(long")[0]


def trace_series(db: str, min_dispatches: int = 10):
    """Maximal runs of consecutive dispatches (in start order) of one kernel
    at one grid, with at least `min_dispatches` dispatches: the series that a
    benchmark times back to back.  Two shapes that launch the same kernel
    with the same grid stay apart here, where a grouping by name and grid
    would average them together."""
    c = _db(db)
    rows = c.execute(
        "select name, grid_x*grid_y*grid_z, workgroup_x*workgroup_y*workgroup_z, duration "
        "from kernels order by start").fetchall()
    runs = []
    for name, grid, wg, dur in rows:
        if runs and runs[-1]["name"] == name and runs[-1]["grid"] == grid:
            runs[-1]["d"].append(dur)
        else:
            runs.append({"name": name, "grid": grid, "block": wg, "d": [dur]})
    return [r for r in runs if len(r["d"]) >= min_dispatches]


def trace_summary(db: str, cmd: str) -> str:
    c = _db(db)
    rows = c.execute(
        "select name, grid_x*grid_y*grid_z, workgroup_x*workgroup_y*workgroup_z, count(*), "
        "avg(duration), min(duration), max(duration), sum(duration) from kernels "
        "group by name, grid_x, grid_y, grid_z order by sum(duration) desc").fetchall()
    out = [f"# rocprofv3 kernel trace summary", "",
           f"command: `{cmd}`", "",
           "## Series of back-to-back dispatches, in launch order", "",
           "Each row is a maximal run of consecutive dispatches of one kernel at one grid "
           "(at least 10): a timed series of the benchmark.", "",
           "| # | kernel | grid (lanes) | block | dispatches | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|---|---|"]
    for i, r in enumerate(trace_series(db)):
        d = sorted(r["d"])
        med = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
        out.append(f"| {i} | `{_short(r['name'])}` | {r['grid']} | {r['block']} | {len(d)} | "
                   f"{sum(d) / len(d) / 1e3:.2f} | {med / 1e3:.2f} | {d[0] / 1e3:.2f} | "
                   f"{d[-1] / 1e3:.2f} |")
    out += ["", "## All dispatches by kernel and grid", "",
            "| kernel | grid (lanes) | block | dispatches | avg us | min us | max us |",
            "|---|---|---|---|---|---|---|"]
    for name, grid, wg, n, avg, mn, mx, _ in rows:
        out.append(f"| `{_short(name)}` | {grid} | {wg} | {n} | {avg / 1e3:.2f} | "
                   f"{mn / 1e3:.2f} | {mx / 1e3:.2f} |")
    has_stats = c.execute("select count(*) from sqlite_master where name = 'top_kernels'").fetchone()[0]
    if has_stats:
        # rocprofv3's own --stats summary (by kernel name over all grids), as it wrote it
        out += ["", "## rocprofv3 --stats (its `top_kernels` table, by kernel name)", "",
                "| kernel | calls | total us | average us | % of kernel time |", "|---|---|---|---|---|"]
        for name, calls, total, avg, pct in c.execute(
                "select name, total_calls, total_duration, average, percentage from top_kernels"):
            out.append(f"| `{_short(name)}` | {calls} | {float(total):.1f} | {float(avg):.3f} | "
                       f"{float(pct):.2f} |")
    return "\n".join(out) + "\n"


def _is_gemm(name: str) -> bool:
    return "tra::" in name and "gemm_" in name


def gemm_kernels(db, counter):
    """[(kernel name, grid lanes, dispatches, mean value)] of the library's
    GEMM kernels in a counters database, and the calibration copy's mean
    reading (the copy of the largest grid)."""
    c = _db(db)
    rows = c.execute(
        "select kernel_name, grid_size, count(*), avg(value) from counters_collection "
        "where counter_name = ? group by kernel_name, grid_size", (counter,)).fetchall()
    copies = [r for r in rows if COPY_KERNEL in r[0]]
    if not copies:
        raise SystemExit(f"{db}: no calibration copy ({COPY_KERNEL})")
    gemm = [r for r in rows if _is_gemm(r[0])]
    if not gemm:
        raise SystemExit(f"{db}: no GEMM kernel")
    return gemm, max(copies, key=lambda r: r[1])[3]


def per_call(kernels):
    """Counter value per GEMM call: every kernel a call launches is dispatched
    once per call, so the call count is the largest dispatch count, and each
    kernel contributes mean x dispatches / calls."""
    calls = max(n for _, _, n, _ in kernels)
    return sum(v * n for _, _, n, v in kernels) / calls, calls


def traffic_summary(fetch_db, write_db, workload, cmd, algorithmic_bytes):
    fk, fcopy = gemm_kernels(fetch_db, "FETCH_SIZE")
    wk, wcopy = gemm_kernels(write_db, "WRITE_SIZE")
    fetch_scale = COPY_BYTES / (fcopy * 1024.0)
    write_scale = COPY_BYTES / (wcopy * 1024.0)
    f_kib, calls = per_call(fk)
    w_kib, _ = per_call(wk)
    read_b = f_kib * 1024.0 * fetch_scale
    write_b = w_kib * 1024.0 * write_scale
    total = read_b + write_b
    lines = [
        "# HBM traffic of one GEMM call from rocprofv3 counters",
        f"# FETCH_SIZE pass: {cmd.format(counter='FETCH_SIZE')}",
        f"# WRITE_SIZE pass: {cmd.format(counter='WRITE_SIZE')}",
        f"# calibration: plain device copy of {COPY_BYTES} bytes in the same runs:",
        f"#   FETCH_SIZE reads {fcopy:.1f} KiB -> scale {fetch_scale:.4f};"
        f" WRITE_SIZE reads {wcopy:.1f} KiB -> scale {write_scale:.4f}",
    ]
    for name, grid, n, v in fk:
        w = [x for x in wk if x[0] == name and x[1] == grid]
        lines.append(f"# kernel: {_short(name)} grid_lanes {grid} dispatches {n}: "
                     f"FETCH_SIZE {v:.1f} KiB, WRITE_SIZE {w[0][3] if w else float('nan'):.1f} KiB")
    lines += [
        f"workload = {workload}",
        f"calls = {calls}",
        f"fetch_size_kib = {f_kib:.1f}",
        f"write_size_kib = {w_kib:.1f}",
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


def drive(workload: str, reps: int, calibration: bool = True) -> None:
    """Runs `workload` through gemm_f32 (the library's choice) 2 + reps
    times on device-resident inputs, after 5 plain device copies of
    COPY_BYTES bytes (the calibration for FETCH_SIZE and WRITE_SIZE)."""
    sys.path.insert(0, ROOT)
    import torch
    import tiling_roofline_analysis_amd as tra
    from tiling_roofline_analysis_amd import inputs
    w = inputs.WORKLOADS[workload]
    A, B = w.make()
    dA = torch.from_numpy(A).to("cuda:0")
    dB = torch.from_numpy(B).to("cuda:0")
    dC = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
    del A, B
    if calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    h = torch.cuda.current_stream().cuda_stream
    print(f"[drive] {workload}: {tra.tra_gemm_describe(tra.AUTO, w.M, w.N, w.K)}",
          file=sys.stderr, flush=True)
    for _ in range(2 + reps):
        st = tra.gemm_f32(w.M, w.N, w.K, dA.data_ptr(), w.K, dB.data_ptr(), w.N, dC.data_ptr(),
                          w.N, h)
        if st != tra.TRA_OK:
            raise tra.TraError(st, "gemm_f32")
    torch.cuda.synchronize()
    print(f"[drive] {workload}: {2 + reps} calls done", file=sys.stderr, flush=True)


def configs_summary(pairs, cmd):
    """Markdown table of the SQ counters (SQ_COUNTERS) of every GEMM kernel of
    each workload, from one `--pmc` run of `drive` per workload."""
    lines = [
        "# SQ counters per dispatch of each configured workload's kernels (rocprofv3 --pmc)", "",
        f"Command, once per workload: `{cmd}`", "",
        "Averages per dispatch. `clk` = GRBM_GUI_ACTIVE / 8 XCDs, the kernel's length in GPU "
        "clocks. SIMD-clocks = 4 SIMDs x 256 CUs x clk.", "",
        "| workload | kernel | grid (lanes) | dispatches | duration us | clk/2.4GHz us | "
        "LDS instr | bank-conflict cycles per LDS instr | LDS wait / wave cycles | VALU instr | "
        "MFMA instr | MFMA busy / SIMD-clocks |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for workload, db in pairs:
        c = _db(db)
        rows = c.execute(
            "select kernel_name, grid_size, counter_name, avg(value), count(*), avg(duration) "
            "from counters_collection group by kernel_name, grid_size, counter_name").fetchall()
        kernels = {}
        for name, grid, cn, v, n, dur in rows:
            if not _is_gemm(name):
                continue
            d = kernels.setdefault((name, grid), {"dispatches": n, "duration_ns": dur})
            d[cn] = v
        for (name, grid), d in kernels.items():
            clk = d.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
            simd_clk = SIMDS_PER_CU * CUS * clk
            lds = d.get("SQ_INSTS_LDS", 0.0)
            conflict = d.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else 0.0
            wc = d.get("SQ_WAVE_CYCLES", 0.0)
            wait = d.get("SQ_WAIT_INST_LDS", 0.0) / wc if wc else 0.0
            busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / simd_clk if simd_clk else 0.0
            lines.append(
                f"| {workload} | `{_short(name)}` | {grid} | {d['dispatches']} | "
                f"{d['duration_ns'] / 1e3:.1f} | {clk / 2.4e3:.1f} | {lds:.4g} | {conflict:.3f} | "
                f"{wait:.3f} | {d.get('SQ_INSTS_VALU', 0.0):.4g} | "
                f"{d.get('SQ_INSTS_MFMA', 0.0):.4g} | {busy:.3f} |")
    lines += ["", f"sources_digest = {all_sources_digest()}"]
    return "\n".join(lines) + "\n"


def ladder_traffic(fetch_db, write_db):
    """Calibrated HBM bytes per launch of every rung of the ladder in two
    `--pmc` runs of bench.py with its ladder, keyed by (rung, workload).
    A rung's launch is recognised by its kernel name and its grid, which
    tra_gemm_describe gives for each configured shape."""
    def rows(db):
        c = _db(db)
        return c.execute(
            "select kernel_name, grid_size, avg(value), count(*) from counters_collection "
            "group by kernel_name, grid_size").fetchall()

    out = {}
    fr, wr = rows(fetch_db), rows(write_db)
    cf = max((r for r in fr if COPY_KERNEL in r[0]), key=lambda r: r[1])
    cw = max((r for r in wr if COPY_KERNEL in r[0]), key=lambda r: r[1])
    fscale, wscale = COPY_BYTES / (cf[2] * 1024.0), COPY_BYTES / (cw[2] * 1024.0)
    for rung, wname, kernel, lanes in ladder_launches():
        f = [r for r in fr if _is_launch(r[0], r[1], kernel, lanes)]
        wrow = [r for r in wr if _is_launch(r[0], r[1], kernel, lanes)]
        if len(f) != 1 or len(wrow) != 1:
            continue
        out[(rung, wname)] = {
            "kernel": kernel, "lanes": lanes, "dispatches": f[0][3],
            "read_bytes": f[0][2] * 1024.0 * fscale, "write_bytes": wrow[0][2] * 1024.0 * wscale}
    return out, fscale, wscale


def ladder_launches():
    """(rung, workload, kernel name, grid in lanes) of every launch that
    bench.py's ladder makes, from tra_gemm_describe at both configured shapes."""
    sys.path.insert(0, ROOT)
    import tiling_roofline_analysis_amd as tra
    from tiling_roofline_analysis_amd import inputs
    for wname in ("uniform1024", "normal4096"):
        w = inputs.WORKLOADS[wname]
        for v in tra.LADDER:
            d = tra.tra_gemm_describe(v, w.M, w.N, w.K)
            kv = dict(x.split("=", 1) for x in d.split() if "=" in x)
            yield (tra.tra_gemm_variant_name(v), wname, kv["kernel"].split("<")[0],
                   int(kv["grid"]) * int(kv["block"]))


def _is_launch(name, grid, kernel, lanes):
    return (kernel + "<" in name or kernel + "(" in name) and grid == lanes


# Counters of one `--pmc` pass over bench.py's ladder (at most 8 SQ and 2 GRBM
# counters fit in one pass).
SQ_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_LDS",
               "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
CUS, XCDS, SIMDS_PER_CU = 256, 8, 4


def ladder_counters(db):
    """Per-dispatch averages of SQ_COUNTERS for every rung of bench.py's
    ladder, keyed by (rung, workload), plus the dispatch duration that the
    same run recorded."""
    c = _db(db)
    rows = c.execute(
        "select kernel_name, grid_size, counter_name, avg(value), count(*), avg(duration) "
        "from counters_collection group by kernel_name, grid_size, counter_name").fetchall()
    out = {}
    for rung, wname, kernel, lanes in ladder_launches():
        mine = [r for r in rows if _is_launch(r[0], r[1], kernel, lanes)]
        if not mine or len({r[0] for r in mine}) != 1:
            continue
        d = {r[2]: r[3] for r in mine}
        d["dispatches"] = mine[0][4]
        d["duration_ns"] = mine[0][5]
        d["kernel"] = kernel
        out[(rung, wname)] = d
    return out


def counters_summary(db, cmd):
    """Markdown table of the SQ counters per rung: what each rung of the
    ladder spends its cycles on. GRBM_GUI_ACTIVE reads the sum over the XCDs;
    divided by their count it is the kernel's length in GPU clocks, which the
    summary checks against the recorded duration at 2.4 GHz."""
    data = ladder_counters(db)
    lines = [
        "# SQ counters per launch of each rung (rocprofv3 --pmc)", "",
        f"Command: `{cmd}`", "",
        "Averages per dispatch. `clk` = GRBM_GUI_ACTIVE / 8 XCDs, the kernel's length in "
        "GPU clocks (`clk / 2.4 GHz` is given beside the duration the same run recorded). "
        "SIMD-clocks = 4 SIMDs x 256 CUs x clk.", "",
        "| rung | workload | kernel | dispatches | duration us | clk/2.4GHz us | LDS instr | "
        "bank-conflict cycles per LDS instr | LDS wait / wave cycles | VALU instr | "
        "VALU instr per SIMD-clock | MFMA instr | MFMA busy / SIMD-clocks |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for (rung, wname), d in data.items():
        clk = d["GRBM_GUI_ACTIVE"] / XCDS
        simd_clk = SIMDS_PER_CU * CUS * clk
        lds = d["SQ_INSTS_LDS"]
        conflict = d["SQ_LDS_BANK_CONFLICT"] / lds if lds else 0.0
        wait = d["SQ_WAIT_INST_LDS"] / d["SQ_WAVE_CYCLES"] if d["SQ_WAVE_CYCLES"] else 0.0
        lines.append(
            f"| {rung} | {wname} | {d['kernel']} | {d['dispatches']} | "
            f"{d['duration_ns'] / 1e3:.1f} | {clk / 2.4e3:.1f} | {lds:.4g} | {conflict:.3f} | "
            f"{wait:.3f} | {d['SQ_INSTS_VALU']:.4g} | {d['SQ_INSTS_VALU'] / simd_clk:.3f} | "
            f"{d['SQ_INSTS_MFMA']:.4g} | {d['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_clk:.3f} |")
    lines += ["", f"sources_digest = {all_sources_digest()}"]
    return "\n".join(lines) + "\n"


def ladder_summary(fetch_db, write_db, cmd):
    from tiling_roofline_analysis_amd import inputs, roofline
    data, fscale, wscale = ladder_traffic(fetch_db, write_db)
    lines = [
        "# HBM traffic per launch of each rung (rocprofv3 counters)", "",
        f"FETCH_SIZE pass: `{cmd.format(counter='FETCH_SIZE')}`", "",
        f"WRITE_SIZE pass: `{cmd.format(counter='WRITE_SIZE')}`", "",
        f"Calibration by a plain device copy of {COPY_BYTES} bytes in the same runs: "
        f"FETCH_SIZE x {fscale:.4f}, WRITE_SIZE x {wscale:.4f}.", "",
        "| rung | workload | kernel | HBM read B | HBM write B | x algorithmic | achieved AI (flop/B) |",
        "|---|---|---|---|---|---|---|"]
    for (rung, wname), d in data.items():
        w = inputs.WORKLOADS[wname]
        alg = roofline.gemm_bytes(w.M, w.N, w.K)
        tot = d["read_bytes"] + d["write_bytes"]
        lines.append(f"| {rung} | {wname} | {d['kernel']} | {d['read_bytes']:.4g} | "
                     f"{d['write_bytes']:.4g} | {tot / alg:.2f} | "
                     f"{roofline.gemm_flops(w.M, w.N, w.K) / tot:.4g} |")
    lines += ["", f"sources_digest = {all_sources_digest()}"]
    return "\n".join(lines) + "\n"


def all_sources_digest() -> str:
    """Digest of the code of every kernel source of the library."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(HERE, "csrc"))):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(HERE, "csrc", f), encoding="utf-8") as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


LADDER_TRAFFIC = os.path.join(PROFILES, "traffic_ladder.md")


def stored_ladder_traffic():
    """{(rung, workload): HBM bytes per launch} from profiles/traffic_ladder.md,
    or {} when it is absent or the kernel sources changed since."""
    if not os.path.exists(LADDER_TRAFFIC):
        return {}
    text = open(LADDER_TRAFFIC).read()
    m = re.search(r"sources_digest = (\w+)", text)
    if not m or m.group(1) != all_sources_digest():
        return {}
    out = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] not in ("rung", "---"):
            try:
                out[(cells[0], cells[1])] = float(cells[3]) + float(cells[4])
            except ValueError:
                pass
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description="summarise rocprofv3 results")
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("fetch_db")
    f.add_argument("write_db")
    f.add_argument("--workload", required=True)
    f.add_argument("--cmd", required=True, help="profiling command with {counter}")
    dr = sub.add_parser("drive")
    dr.add_argument("workload")
    dr.add_argument("--reps", type=int, default=20)
    dr.add_argument("--no-calibration", action="store_true")
    cf = sub.add_parser("configs")
    cf.add_argument("--cmd", required=True, help="the profiling command")
    cf.add_argument("pairs", nargs="+", help="WORKLOAD=DB")
    lad = sub.add_parser("ladder")
    lad.add_argument("fetch_db")
    lad.add_argument("write_db")
    lad.add_argument("--cmd", required=True, help="profiling command with {counter}")
    cnt = sub.add_parser("counters")
    cnt.add_argument("db")
    cnt.add_argument("--cmd", required=True, help="the profiling command")
    args = ap.parse_args(argv)
    if args.what == "trace":
        sys.stdout.write(trace_summary(args.db, args.cmd))
    elif args.what == "counters":
        sys.stdout.write(counters_summary(args.db, args.cmd))
    elif args.what == "ladder":
        sys.path.insert(0, ROOT)
        sys.stdout.write(ladder_summary(args.fetch_db, args.write_db, args.cmd))
    elif args.what == "drive":
        drive(args.workload, args.reps, not args.no_calibration)
    elif args.what == "configs":
        pairs = [tuple(x.split("=", 1)) for x in args.pairs]
        sys.stdout.write(configs_summary(pairs, args.cmd))
    else:
        sys.path.insert(0, ROOT)
        from tiling_roofline_analysis_amd import inputs, roofline
        w = inputs.WORKLOADS[args.workload]
        sys.stdout.write(traffic_summary(args.fetch_db, args.write_db, args.workload, args.cmd,
                                         roofline.gemm_bytes(w.M, w.N, w.K)))


if __name__ == "__main__":
    main()
