#!/usr/bin/env python3
"""FP32 GEMM benchmark on one MI355X: TFLOP/s and fraction of the roofline.

One step is one C = A x B through the C ABI (libtra_gemm.so) on device-
resident inputs.  The headline workload is M = N = K = 1024 with seeded
uniform[-1, 1) inputs (50 timed launches after warm-up, as the page "GEMM
kernel test code & optimization (1024^3 experiment)" times its kernels);
M = N = K = 4096 with normal(0, 1) inputs is reported beside it as
"secondary".  Every rung of the kernel ladder is also timed on both shapes
("ladder"), and the library's own choice on the ragged and tall-skinny shapes
and on one GPU's slab of the two large shapes split over 8 GPUs ("shapes").

Timing: HIP events recorded on the stream the kernels are launched on
(torch's current stream), around `--steps` back-to-back launches, after
`--warmup` launches; per-launch event pairs give min/median.  Before the
warm-up launches of each headline shape, the same GEMM runs untimed for
`--warm-seconds` (0.5 s) so that timing starts at the GPU's sustained
clocks rather than while they ramp up.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP32 GEMM TFLOP/s and % of roofline at 1024³ and 4096³, 1× MI355X"
PRIMARY = "uniform1024"
SECONDARY = "normal4096"
# Timed for context (`shapes` in the JSON line): the ragged and tall-skinny
# shapes, and the per-GPU slabs of 4096^3 (512 rows of C) and of the
# tall-skinny product (2048 of K) when split over 8 GPUs.
OTHER_SHAPES = ("ragged", "tall", "rowslab4096", "kslab_tall")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_variant(tra, torch, variant, w, dA, dB, dC, steps, warmup, warm_seconds=0.0):
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    pa, pb, pc = dA.data_ptr(), dB.data_ptr(), dC.data_ptr()
    M, N, K = w.M, w.N, w.K
    fn = tra.load().gemm_f32_variant

    def launch():
        st = fn(variant, M, N, K, pa, K, pb, N, pc, N, handle)
        if st != tra.TRA_OK:
            raise tra.TraError(st, "gemm_f32_variant")

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    if warm_seconds > 0:
        # bring the GPU to its sustained clocks with the same launch, untimed
        t_end = time.perf_counter() + warm_seconds
        while time.perf_counter() < t_end:
            for _ in range(20):
                launch()
            torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        launch()
    end.record(stream)
    end.synchronize()
    avg_ms = start.elapsed_time(end) / steps
    # per-launch pairs (a separate pass, so the loop above has no extra events)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(min(steps, 50))]
    for s, e in pairs:
        s.record(stream)
        launch()
        e.record(stream)
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in pairs]
    return avg_ms, min(per), statistics.median(per)


def measure_roofs(tra, torch):
    """The two roofs measured on this device with the library's probes: HBM
    bandwidth from a 1 GiB streaming copy (larger than the 256 MB last-level
    cache), the FP32 MFMA and FP32 VALU (no packed FP32) peaks."""
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream

    def timed(call, reps):
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            st = call()
            if st != tra.TRA_OK:
                raise tra.TraError(st, "probe")
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    n = 256 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    t = timed(lambda: tra.tra_probe_copy_f32(n, src.data_ptr(), dst.data_ptr(), h), 5)
    out["hbm_copy_tbps"] = round(tra.tra_probe_work(tra.PROBE_COPY, n) / t / 1e12, 3)
    del src, dst
    torch.cuda.empty_cache()
    sink = torch.empty(tra.PROBE_SINK_FLOATS, dtype=torch.float32, device="cuda:0")
    it = 20000
    t = timed(lambda: tra.tra_probe_mfma_f32(it, sink.data_ptr(), h), 3)
    out["mfma_fp32_tflops"] = round(tra.tra_probe_work(tra.PROBE_MFMA, it) / t / 1e12, 2)
    it = 100000
    t = timed(lambda: tra.tra_probe_fma_f32(it, sink.data_ptr(), h), 3)
    out["valu_fp32_tflops"] = round(tra.tra_probe_work(tra.PROBE_FMA, it) / t / 1e12, 2)
    out["ridge_flop_per_byte"] = round(out["mfma_fp32_tflops"] / out["hbm_copy_tbps"], 2)
    # the floor under a one-launch GEMM: back-to-back launches of an empty
    # kernel on as many workgroups as the 1024^3 GEMM launches
    t = timed(lambda: tra.tra_probe_launch(256, h), 500)
    out["launch_floor_us"] = round(t * 1e6, 2)
    return out


def host_inclusive(tra, torch, w, reps=5):
    """Host-to-host time of one product, as page "[AutoMine++] #2 matmul
    trial and error" timed its SYCL routine (section "Implementing with SYCL
    (iGPU) + performance comparison"): device buffers, host-to-device copies
    of A and B, the GEMM, the copy of C back, all inside the clock.  Device buffers come
    from torch's caching allocator (cached after the first rep, which is
    not timed).  Pageable and pinned host memory are both timed."""
    A, B = w.make()
    out = {}
    for mode in ("pageable", "pinned"):
        hA, hB = torch.from_numpy(A), torch.from_numpy(B)
        hC = torch.empty((w.M, w.N), dtype=torch.float32)
        if mode == "pinned":
            hA, hB, hC = hA.pin_memory(), hB.pin_memory(), hC.pin_memory()
        times = []
        for r in range(reps + 1):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            dA = hA.to("cuda:0", non_blocking=(mode == "pinned"))
            dB = hB.to("cuda:0", non_blocking=(mode == "pinned"))
            dC = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
            tra.matmul(dA, dB, dC)
            hC.copy_(dC, non_blocking=(mode == "pinned"))
            torch.cuda.synchronize()
            if r > 0:
                times.append(time.perf_counter() - t0)
            del dA, dB, dC
        t = statistics.median(times)
        out[f"{mode}_ms"] = round(t * 1e3, 4)
        out[f"{mode}_tflops"] = round(w.flops / t / 1e12, 3)
    out["bytes_over_pcie"] = 4 * (w.M * w.K + w.K * w.N + w.M * w.N)
    return out


def torch_matmul(torch, w, steps):
    """torch.matmul in strict FP32 (ROCm's vendor GEMM) on the same device-
    resident inputs, timed like the library: context, not the product."""
    torch.backends.cuda.matmul.allow_tf32 = False
    A, B = w.make()
    dA = torch.from_numpy(A).to("cuda:0")
    dB = torch.from_numpy(B).to("cuda:0")
    dC = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(5):
        torch.matmul(dA, dB, out=dC)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        torch.matmul(dA, dB, out=dC)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"ms": round(ms, 5), "tflops": round(w.flops / ms / 1e9, 3)}


def numpy_matmul(w):
    """numpy's float32 matmul (the host BLAS) on the same inputs: the
    comparison page "[AutoMine++] #2 matmul trial and error" plans in its
    section "Wrap-up"."""
    import numpy as np
    A, B = w.make()
    np.matmul(A, B)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        np.matmul(A, B)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"ms": round(t * 1e3, 3), "tflops": round(w.flops / t / 1e12, 4)}


def time_cold(tra, torch, w, dA, dB, dC, launches=20):
    """Per-launch time with the caches flushed before each launch: a 512 MiB
    buffer (twice the 256 MB last-level cache) is read and written between
    launches, outside the event pair, so A and B come from HBM."""
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    fn = tra.load().gemm_f32_variant
    scratch = torch.zeros(128 << 20, dtype=torch.float32, device="cuda:0")
    pairs = []
    for _ in range(launches):
        scratch.add_(1.0)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = fn(tra.AUTO, w.M, w.N, w.K, dA.data_ptr(), w.K, dB.data_ptr(), w.N,
                dC.data_ptr(), w.N, handle)
        if st != tra.TRA_OK:
            raise tra.TraError(st, "gemm_f32_variant")
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    del scratch
    per = sorted(a.elapsed_time(b) for a, b in pairs[1:])
    med = statistics.median(per)
    return {"median_ms": round(med, 5), "min_ms": round(per[0], 5),
            "tflops": round(w.flops / med / 1e9, 3), "launches": len(per)}


def shape_label(w):
    return f"M=N=K={w.M}" if w.M == w.N == w.K else f"M={w.M} N={w.N} K={w.K}"


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# The oracle timed beside each configuration: (workload, timed runs after one
# warm-up run (0: a single run), also on one thread).  The small shapes take
# 1 warm-up and 3 timed runs on all cores and on one thread; the large ones
# one run on all cores (4096^3 is 6.9e10 binary64 multiply-adds: about 20 s
# on 16 cores).
ORACLE_CONFIGS = (("int256", 3, True), ("uniform1024", 3, True), ("normal4096", 0, False),
                  ("ragged", 0, False), ("tall", 0, False))


def cpu_baseline_configs(workloads):
    """Part of the CPU-baseline leg: the CPU oracle on every configured shape,
    beside the GPU numbers, with a wall clock around each call, as page
    "[AutoMine++] #2 matmul trial and error" times its CPU loop (section
    "Intuitive implementation (by CPU)")."""
    import oracle
    every = oracle.default_threads()
    out = {"host_cpus": os.cpu_count(), "cpu_model": cpu_model(), "threads_all_cores": every,
           "configs": {}}
    for name, runs, one_thread in ORACLE_CONFIGS:
        w = workloads[name]
        A, B = w.make()
        entry = {"workload": f"{w.M}x{w.N}x{w.K}, {w.what}"}
        for threads in (every, 1) if one_thread else (every,):
            if runs:
                oracle.gemm(A, B, nthreads=threads)   # warm-up, untimed
            times = []
            for _ in range(max(1, runs)):
                t0 = time.perf_counter()
                oracle.gemm(A, B, nthreads=threads)
                times.append(time.perf_counter() - t0)
            t = statistics.median(times)
            entry[f"threads_{threads}"] = {
                "runs_s": [round(x, 4) for x in times], "median_s": round(t, 4),
                "gflops": round(w.flops / t / 1e9, 3)}
            log(f"[oracle] {name} on {threads} thread(s): {entry[f'threads_{threads}']}")
        out["configs"][name] = entry
        del A, B
    return out


def cpu_baseline(w, seconds=10.0):
    """The CPU oracle on the full headline product, on the host's cores,
    repeated for about `seconds` of wall time (at least 3 runs); the median
    run is reported."""
    import oracle
    A, B = w.make()
    threads = oracle.default_threads()
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t_all < seconds:
        t0 = time.perf_counter()
        oracle.gemm(A, B, nthreads=threads)
        times.append(time.perf_counter() - t0)
    total = time.perf_counter() - t_all
    t = statistics.median(times)
    return {
        "value": w.flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": (f"full {w.M}x{w.N}x{w.K} product ({w.what}), binary64 triple loop, "
                   f"{len(times)} runs over {total:.1f} s, median run {t:.3f} s"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ladder", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-roofs", action="store_true", help="skip the roof probes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times (scales HBM counters)")
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed launches of the headline GEMM before its warm-up steps, so "
                         "the GPU runs at its sustained clocks when timing starts")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timing of the two headline shapes")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip timing the ragged, tall-skinny and per-GPU-slab shapes")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip host-inclusive timing and the torch / numpy comparisons")
    ap.add_argument("--config", default=PRIMARY,
                    help="the headline workload (default %(default)s; the others: "
                         "int256, const256, int1024, normal4096, ragged, tall, rowslab4096, "
                         "kslab_tall)")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the random inputs (A takes SEED, B SEED + 1) in place of "
                         "each workload's own")
    ap.add_argument("--no-oracle-configs", action="store_true",
                    help="skip timing the CPU oracle on every configured shape")
    ap.add_argument("--plot", metavar="SVG", help="write the roofline chart of the ladder here")
    ap.add_argument("--plot-table", metavar="MD", help="write the chart's points as a table here")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this GEMM has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import torch
    import tiling_roofline_analysis_amd as tra
    from tiling_roofline_analysis_amd import inputs
    from tiling_roofline_analysis_amd import roofline as rl
    from tiling_roofline_analysis_amd.profiling import (source_digest, stored_ladder_traffic,
                                                        stored_traffic)

    if args.config not in inputs.WORKLOADS:
        ap.error(f"--config: no workload {args.config!r}")
    # the workloads, with the random ones reseeded if asked
    workloads = {name: (dataclasses.replace(w, seed=args.seed, what=f"{w.what.split(' seeds')[0]} "
                                                                  f"seeds {args.seed}/{args.seed + 1}")
                        if args.seed is not None and w.seed is not None else w)
                 for name, w in inputs.WORKLOADS.items()}
    primary = args.config
    secondary = None if args.no_secondary or args.config == SECONDARY else SECONDARY
    if not os.path.exists(tra.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    tra.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    def measure(name, steps, warmup, ladder, cold=False):
        w = workloads[name]
        A, B = w.make()
        dA = torch.from_numpy(A).to("cuda:0")
        dB = torch.from_numpy(B).to("cuda:0")
        dC = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda:0")
        log(f"[{name}] {tra.tra_gemm_describe(tra.AUTO, w.M, w.N, w.K)}")
        avg, mn, med = time_variant(tra, torch, tra.AUTO, w, dA, dB, dC, steps, warmup,
                                    args.warm_seconds)
        rep = rl.gemm_roofline(w.M, w.N, w.K, avg * 1e-3)
        log(f"[{name}] auto(mfma): {avg * 1e3:.2f} us/launch (min {mn * 1e3:.2f}, "
            f"median {med * 1e3:.2f}) = {rep['tflops']:.2f} TFLOP/s, "
            f"{100 * rep['frac_of_roof']:.1f}% of roof")
        out = {"w": w, "avg_ms": avg, "min_ms": mn, "median_ms": med, "rep": rep, "ladder": {}}
        if cold:
            out["cold"] = time_cold(tra, torch, w, dA, dB, dC)
            log(f"[{name}] cold caches: {out['cold']}")
        if ladder:
            for v in tra.LADDER:
                # keep each rung's timed region to about half a second
                probe, _, _ = time_variant(tra, torch, v, w, dA, dB, dC, 1, 1)
                st = max(3, min(steps, int(500.0 / max(probe, 1e-3))))
                a2, m2, md2 = time_variant(tra, torch, v, w, dA, dB, dC, st, 1)
                r2 = rl.gemm_roofline(w.M, w.N, w.K, a2 * 1e-3)
                name_v = tra.tra_gemm_variant_name(v)
                out["ladder"][name_v] = {
                    "ms": round(a2, 5), "tflops": round(r2["tflops"], 3),
                    "frac_of_fp32_peak": round(r2["tflops"] / rl.PEAK_FP32_MFMA_TFLOPS, 4),
                    "unit": "mfma" if v == tra.MFMA else "valu", "steps": st}
                log(f"[{name}] {name_v:12s} {a2 * 1e3:10.2f} us  {r2['tflops']:8.2f} TFLOP/s")
        del dA, dB, dC
        torch.cuda.empty_cache()
        return out

    if args.copy_calibration:
        # A plain device-to-device copy of known size: 256 MiB read, 256 MiB
        # written per launch.  Profilers' FETCH_SIZE / WRITE_SIZE readings of
        # this kernel calibrate the same counters on the GEMM kernels.
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[copy-calibration] 5 x copy of {src.numel() * 4} bytes")
        del src, dst
        torch.cuda.empty_cache()

    t_wall = time.perf_counter()
    prim = measure(primary, args.steps, args.warmup, not args.no_ladder, not args.no_cold)
    sec = None if secondary is None else measure(secondary, args.steps, args.warmup,
                                                 not args.no_ladder, not args.no_cold)
    shapes = {}
    if not args.no_shapes:
        # Context beside the headline: the other large shapes and one GPU's
        # share of the two large shapes split over 8 GPUs, each through AUTO.
        for name in (x for x in OTHER_SHAPES if x != primary):
            m = measure(name, args.steps, args.warmup, False)
            ws, rep = m["w"], m["rep"]
            shapes[name] = {
                "workload": f"FP32 GEMM {ws.M}x{ws.N}x{ws.K} row-major, {ws.what}",
                "value": round(rep["tflops"], 3), "unit": "TFLOP/s",
                "ms_per_step": round(m["avg_ms"], 5), "min_ms": round(m["min_ms"], 5),
                "frac_of_fp32_peak": round(rep["tflops"] / rl.PEAK_FP32_MFMA_TFLOPS, 4),
                "frac_of_hbm_floor": round(rep["frac_of_hbm_floor"], 4),
                "kernel": tra.tra_gemm_describe(tra.AUTO, ws.M, ws.N, ws.K),
                "traffic": stored_traffic(name)}
    gpu_wall = time.perf_counter() - t_wall
    roofs = None
    if not args.no_roofs:
        roofs = measure_roofs(tra, torch)
        log(f"[roofs] measured: {roofs}")
        # each rung against the measured roof of the unit it runs on
        for m in (prim, sec):
            for entry in (m or {}).get("ladder", {}).values():
                roof = roofs["mfma_fp32_tflops" if entry["unit"] == "mfma" else "valu_fp32_tflops"]
                entry["frac_of_measured_unit_roof"] = round(entry["tflops"] / roof, 4)

    def roofline_obj(m, workload):
        rep = m["rep"]
        return {"bound": "mfma", "achieved": round(rep["tflops"], 3),
                "peak": rl.PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(rep["tflops"] / rl.PEAK_FP32_MFMA_TFLOPS, 4),
                "traffic": stored_traffic(workload)}

    w = prim["w"]
    line = {
        "metric": METRIC,
        "value": round(prim["rep"]["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["avg_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"FP32 GEMM {shape_label(w)} row-major, {w.what}",
                   "M": w.M, "N": w.N, "K": w.K, "kernel": tra.tra_gemm_describe(tra.AUTO, w.M, w.N, w.K)},
        "roofline": roofline_obj(prim, primary),
        "detail": {
            "min_ms": round(prim["min_ms"], 5), "median_ms": round(prim["median_ms"], 5),
            "ai_flop_per_byte": round(prim["rep"]["ai"], 2),
            "algorithmic_bytes": prim["rep"]["bytes"],
            "source_digest": source_digest(), "gpu_wall_s": round(gpu_wall, 2),
            "device": (f"{torch.cuda.get_device_name(0)} "
                       f"({torch.cuda.get_device_properties(0).gcnArchName.split(':')[0]})"),
            "measured_roofs": roofs,
        },
    }
    if "cold" in prim:
        line["detail"]["cold"] = {primary: prim["cold"]}
        if sec is not None:
            line["detail"]["cold"][secondary] = sec["cold"]
    if prim["ladder"]:
        line["ladder"] = {primary: prim["ladder"]}
    if sec is not None:
        ws = sec["w"]
        line["secondary"] = {
            "workload": f"FP32 GEMM {shape_label(ws)} row-major, {ws.what}",
            "value": round(sec["rep"]["tflops"], 3), "unit": "TFLOP/s",
            "ms_per_step": round(sec["avg_ms"], 5), "min_ms": round(sec["min_ms"], 5),
            "kernel": tra.tra_gemm_describe(tra.AUTO, ws.M, ws.N, ws.K),
            "roofline": roofline_obj(sec, secondary),
        }
        if sec["ladder"]:
            line.setdefault("ladder", {})[secondary] = sec["ladder"]
    if shapes:
        line["shapes"] = shapes
    if not args.no_compare:
        comp = {}
        for name in (primary,) + (() if secondary is None else (secondary,)):
            wc = workloads[name]
            comp[name] = {"host_inclusive": host_inclusive(tra, torch, wc),
                          "torch_matmul_fp32": torch_matmul(torch, wc, args.steps)}
            log(f"[{name}] host-inclusive {comp[name]['host_inclusive']}; "
                f"torch.matmul {comp[name]['torch_matmul_fp32']}")
            torch.cuda.empty_cache()
        comp[primary]["numpy_matmul_fp32"] = numpy_matmul(workloads[primary])
        log(f"[{primary}] numpy {comp[primary]['numpy_matmul_fp32']}")
        line["detail"]["compare"] = comp
    if args.plot or args.plot_table:
        rl.write_chart(line, stored_ladder_traffic(), args.plot, args.plot_table)
    if not args.no_cpu_baseline:
        log("[cpu_baseline] timing the oracle ...")
        line["cpu_baseline"] = cpu_baseline(workloads[primary])
        log(f"[cpu_baseline] {line['cpu_baseline']['value'] * 1e3:.3f} GFLOP/s")
        if not args.no_oracle_configs:
            line["detail"]["cpu_oracle"] = cpu_baseline_configs(workloads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
