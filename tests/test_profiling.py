"""Host-side tests of the rocprofv3 summaries (profiling.py) on small
synthetic databases with the rocpd tables the summaries read."""
import sqlite3

import pytest

import tiling_roofline_analysis_amd as tra
from tiling_roofline_analysis_amd import inputs, profiling


def _counters_db(path, rows):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, grid_size int, "
              "counter_name text, value real, duration real)")
    c.executemany("insert into counters_collection values (?,?,?,?,?)", rows)
    c.commit()
    c.close()


def _launches():
    return list(profiling.ladder_launches())


def _kernel_name(kernel):
    return f"void tra::{kernel}<tra::Tile<1, 2> >(long, long, long, float const*)"


def test_ladder_launches_cover_every_rung_at_both_shapes():
    got = _launches()
    assert len(got) == 2 * len(tra.LADDER)
    for rung, wname, kernel, lanes in got:
        w = inputs.WORKLOADS[wname]
        assert kernel.startswith("gemm_")
        assert lanes > 0 and lanes % 64 == 0
        assert rung in [tra.tra_gemm_variant_name(v) for v in tra.LADDER]
        assert w.M * w.N > 0


def _trace_db(path, rows):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, grid_x int, grid_y int, grid_z int, "
              "workgroup_x int, workgroup_y int, workgroup_z int, start int, duration real)")
    c.executemany("insert into kernels values (?,?,?,?,?,?,?,?,?)", rows)
    c.commit()
    c.close()


def test_trace_summary(tmp_path):
    db = tmp_path / "t.db"
    _trace_db(db, [("k1(long)", 256, 1, 1, 256, 1, 1, t, d)
                   for t, d in ((0, 1000.0), (5000, 3000.0))]
              + [("k2(long)", 64, 1, 1, 64, 1, 1, 9000, 500.0)])
    text = profiling.trace_summary(str(db), "cmd")
    by_kernel = text.split("## All dispatches")[1]
    line = [x for x in by_kernel.splitlines() if "`k1`" in x][0]
    cells = [x.strip() for x in line.strip("|").split("|")]
    assert cells[1:] == ["256", "256", "2", "2.00", "1.00", "3.00"]
    # ordered by total time: k1 (4 us) before k2 (0.5 us)
    assert by_kernel.index("`k1`") < by_kernel.index("`k2`")


def test_trace_series_split_one_kernel_between_two_shapes(tmp_path):
    # one kernel at one grid in two timed series with another kernel between
    # them (two shapes that share a tile class): the series stay apart
    db = tmp_path / "s.db"
    rows, t = [], 0
    for dur, n in ((20_000.0, 30), (40_000.0, 12)):
        for _ in range(n):
            rows.append(("gemm(long)", 65536, 1, 1, 256, 1, 1, t, dur))
            t += 100_000
        rows.append(("other(long)", 64, 1, 1, 64, 1, 1, t, 1.0))
        t += 100_000
    rows.append(("gemm(long)", 65536, 1, 1, 256, 1, 1, t, 1e6))   # a lone dispatch
    _trace_db(db, rows)
    series = profiling.trace_series(str(db))
    assert [len(r["d"]) for r in series] == [30, 12]
    assert [sum(r["d"]) / len(r["d"]) for r in series] == [20_000.0, 40_000.0]
    text = profiling.trace_summary(str(db), "cmd")
    first = text.split("## All dispatches")[0]
    assert "| 0 | `gemm` | 65536 | 256 | 30 | 20.00 | 20.00 | 20.00 | 20.00 |" in first
    assert "| 1 | `gemm` | 65536 | 256 | 12 | 40.00 |" in first


def test_ladder_traffic_scales_by_the_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "f.db", tmp_path / "w.db"
    # the copy's counters read half and all of what it moved
    frows = [(copy, 1 << 20, "FETCH_SIZE", profiling.COPY_BYTES / 2048.0, 0.0)]
    wrows = [(copy, 1 << 20, "WRITE_SIZE", profiling.COPY_BYTES / 1024.0, 0.0)]
    for i, (rung, wname, kernel, lanes) in enumerate(_launches()):
        frows.append((_kernel_name(kernel), lanes, "FETCH_SIZE", 100.0 + i, 0.0))
        wrows.append((_kernel_name(kernel), lanes, "WRITE_SIZE", 10.0 + i, 0.0))
    _counters_db(fetch, frows)
    _counters_db(write, wrows)
    data, fs, ws = profiling.ladder_traffic(str(fetch), str(write))
    assert fs == pytest.approx(2.0) and ws == pytest.approx(1.0)
    assert len(data) == len(_launches())
    for i, (rung, wname, kernel, lanes) in enumerate(_launches()):
        d = data[(rung, wname)]
        assert d["read_bytes"] == pytest.approx((100.0 + i) * 1024 * 2)
        assert d["write_bytes"] == pytest.approx((10.0 + i) * 1024)


def test_counters_summary_ratios(tmp_path):
    db = tmp_path / "c.db"
    rows = []
    clk = 1000.0
    for rung, wname, kernel, lanes in _launches():
        v = {"GRBM_GUI_ACTIVE": 8 * clk, "SQ_INSTS_LDS": 400.0, "SQ_LDS_BANK_CONFLICT": 100.0,
             "SQ_WAIT_INST_LDS": 30.0, "SQ_WAVE_CYCLES": 300.0, "SQ_INSTS_VALU": 1024.0 * clk,
             "SQ_INSTS_MFMA": 7.0, "SQ_VALU_MFMA_BUSY_CYCLES": 512.0 * clk,
             "SQ_BUSY_CYCLES": 1.0}
        rows += [(_kernel_name(kernel), lanes, n, x, 2400.0) for n, x in v.items()]
    # a launch of another grid must not be mistaken for a rung
    rows.append((_kernel_name("gemm_naive_f32"), 3, "SQ_INSTS_LDS", 1e9, 1.0))
    _counters_db(db, rows)
    got = profiling.ladder_counters(str(db))
    assert len(got) == len(_launches())
    text = profiling.counters_summary(str(db), "the command")
    assert "the command" in text
    body = [x for x in text.splitlines() if x.startswith("| ") and "---" not in x][1:]
    assert len(body) == len(_launches())
    for line in body:
        cells = [x.strip() for x in line.strip("|").split("|")]
        # duration 2.4 us; clk / 2.4 GHz = 1000 / 2400 us; 400 LDS instructions
        assert cells[4:8] == ["2.4", "0.4", "400", "0.250"]
        # LDS wait share, VALU per SIMD-clock (1024 SIMDs), MFMA busy share
        assert cells[8] == "0.100"
        assert cells[10] == "1.000"
        assert cells[12] == "0.500"


def test_traffic_summary_adds_the_kernels_of_one_call(tmp_path):
    # a split call launches two kernels (parts and fixup), each dispatched
    # once per call; torch's own kernels are left out, and the copy scales
    copy = "__amd_rocclr_copyBuffer"
    parts = "void tra::(anonymous namespace)::gemm_mfma_f32_parts<tra::Tile<64> >(long)"
    fixup = "void tra::(anonymous namespace)::gemm_mfma_f32_fixup<tra::Tile<64> >(long)"
    fetch, write = tmp_path / "f.db", tmp_path / "w.db"
    _counters_db(fetch, [(copy, 1 << 20, "FETCH_SIZE", profiling.COPY_BYTES / 2048.0, 0.0)]
                 + [(parts, 1000, "FETCH_SIZE", 300.0, 0.0)] * 12
                 + [(fixup, 64, "FETCH_SIZE", 20.0, 0.0)] * 12
                 + [("void at::native::fill_kernel(long)", 64, "FETCH_SIZE", 1e6, 0.0)])
    _counters_db(write, [(copy, 1 << 20, "WRITE_SIZE", profiling.COPY_BYTES / 1024.0, 0.0)]
                 + [(parts, 1000, "WRITE_SIZE", 50.0, 0.0)] * 12
                 + [(fixup, 64, "WRITE_SIZE", 8.0, 0.0)] * 12)
    text = profiling.traffic_summary(str(fetch), str(write), "ragged", "cmd {counter}", 1000)
    kv = dict(x.split(" = ") for x in text.splitlines() if " = " in x and not x.startswith("#"))
    assert kv["calls"] == "12"
    assert float(kv["hbm_read_bytes_per_launch"]) == pytest.approx(320.0 * 1024 * 2)
    assert float(kv["hbm_write_bytes_per_launch"]) == pytest.approx(58.0 * 1024)
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx(320.0 * 2048 + 58.0 * 1024)
    assert kv["source_digest"] == profiling.source_digest()
    assert "cmd FETCH_SIZE" in text and "cmd WRITE_SIZE" in text


def test_configs_summary_one_row_per_kernel(tmp_path):
    db = tmp_path / "c.db"
    k = "void tra::(anonymous namespace)::gemm_mfma_f32<tra::Tile<64> >(long)"
    clk = 1000.0
    v = {"GRBM_GUI_ACTIVE": 8 * clk, "SQ_INSTS_LDS": 400.0, "SQ_LDS_BANK_CONFLICT": 0.0,
         "SQ_WAIT_INST_LDS": 30.0, "SQ_WAVE_CYCLES": 300.0, "SQ_INSTS_VALU": 5.0,
         "SQ_INSTS_MFMA": 7.0, "SQ_VALU_MFMA_BUSY_CYCLES": 512.0 * clk}
    _counters_db(db, [(k, 65536, n, x, 2400.0) for n, x in v.items()]
                 + [("void at::native::copy(long)", 64, "SQ_INSTS_LDS", 9.0, 1.0)])
    text = profiling.configs_summary([("tall", str(db))], "the cmd")
    body = [x for x in text.splitlines() if x.startswith("| tall")]
    assert len(body) == 1
    cells = [x.strip() for x in body[0].strip("|").split("|")]
    assert cells[2:9] == ["65536", "1", "2.4", "0.4", "400", "0.000", "0.100"]
    assert cells[11] == "0.500"
