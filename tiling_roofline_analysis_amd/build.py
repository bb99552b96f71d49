"""Build libtra_gemm.so (gfx950 HIP) in-tree with hipcc.

Each source compiles to an object in parallel, then one link makes the shared
library next to this file.  Always rebuilds.  Packed-FP32 instructions are
disabled for device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtra_gemm.so")
# The same sources built with TRA_LDS_POISON=1 (every kernel fills its LDS
# with NaN before use), loaded only by the tests.
POISON_LIB = os.path.join(HERE, "libtra_gemm_poison.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["tra_gemm.hip", "gemm_naive.hip", "gemm_lds_tiled.hip", "gemm_regblock.hip",
           "gemm_mfma.hip", "probes.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str, poison: bool = False) -> str:
    out_dir = os.path.join(BUILD_DIR, "poison") if poison else BUILD_DIR
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    defs = ["-DTRA_LDS_POISON=1"] if poison else []
    cmd = [hipcc(), *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build_library(jobs: int | None = None, poison: bool = False) -> str:
    """Build libtra_gemm.so, or with poison=True the test library
    libtra_gemm_poison.so."""
    out = POISON_LIB if poison else LIB
    os.makedirs(os.path.join(BUILD_DIR, "poison") if poison else BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, poison), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(), file=sys.stderr)
    print(build_library(poison=True), file=sys.stderr)
