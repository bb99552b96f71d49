"""The workgroup -> tile maps of the tiled rungs, checked on the host (no
GPU): tests/tile_maps_check.hip includes the kernels' own header and
compares the 32-bit maps with the 64-bit ones over many grid shapes, and
checks that each map is a bijection (a wrong map would leave tiles of C
unwritten or written twice)."""
from __future__ import annotations

import os
import subprocess

from tiling_roofline_analysis_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tile_maps_on_host(tmp_path):
    exe = str(tmp_path / "tile_maps_check")
    cmd = [build.hipcc(), *build.FLAGS, os.path.join(HERE, "tile_maps_check.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
