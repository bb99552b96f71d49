"""The roof probes on the GPU: the copy probe copies exactly (including a
tail that is not a multiple of 4), the compute probes run, and the measured
roofs are plausible for an MI355X (not a performance assertion: loose
bounds only)."""
import numpy as np
import pytest

import tiling_roofline_analysis_amd as tra

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available()
    tra.load()


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 1 << 20, (1 << 20) + 3])
def test_copy_probe_copies(n):
    import torch
    src = torch.arange(n, dtype=torch.float32, device="cuda:0") * 0.5 - 7.0
    dst = torch.full((n + 4,), -1.0, device="cuda:0")
    st = tra.tra_probe_copy_f32(n, src.data_ptr(), dst.data_ptr(), None)
    assert st == tra.TRA_OK
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert torch.all(dst[n:] == -1.0)


def test_compute_probes_run():
    import torch
    sink = torch.full((tra.PROBE_SINK_FLOATS,), float("nan"), device="cuda:0")
    assert tra.tra_probe_mfma_f32(10, sink.data_ptr(), None) == tra.TRA_OK
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    sink.fill_(float("nan"))
    assert tra.tra_probe_fma_f32(10, sink.data_ptr(), None) == tra.TRA_OK
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()


def test_launch_probe_runs():
    import torch
    for wgs in (1, 256, 4096):
        assert tra.tra_probe_launch(wgs, None) == tra.TRA_OK
    torch.cuda.synchronize()


def test_measured_roofs_plausible():
    import torch
    import bench
    r = bench.measure_roofs(tra, torch)
    assert 2.0 < r["hbm_copy_tbps"] < 9.0
    assert 60.0 < r["mfma_fp32_tflops"] < 170.0
    assert 20.0 < r["valu_fp32_tflops"] < 170.0
    assert 0.5 < r["launch_floor_us"] < 50.0
