"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tra_gemm.hip (argument checks, plans, describe, workspace sizes) is compiled
with both sanitizers on its host side only (device code is never
instrumented), linked with the other kernel sources into a separate library,
and driven by tests/abi_host_check.c, itself built with the sanitizers.  The
driver makes only calls the host answers, so this runs without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from tiling_roofline_analysis_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"
# host-side sanitizers only: each flag goes to the host compilation
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
HOST_SAN += "-Xarch_host -fno-sanitize-recover=undefined".split()
DRIVER_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not os.path.exists(CLANG) or shutil.which("nm") is None:
        pytest.skip("ROCm clang not found")
    d = tmp_path_factory.mktemp("san")
    objs = []
    for src in build.SOURCES:
        stem = os.path.splitext(src)[0] + ".o"
        prebuilt = os.path.join(build.BUILD_DIR, stem)
        if src != "tra_gemm.hip" and os.path.exists(prebuilt):
            objs.append(prebuilt)   # kernel objects from the product build
            continue
        obj = str(d / stem)
        flags = build.FLAGS + (HOST_SAN if src == "tra_gemm.hip" else [])
        _run([build.hipcc(), *flags, "-g", "-c", os.path.join(build.CSRC, src), "-o", obj])
        objs.append(obj)
    lib = str(d / "libtra_gemm_san.so")
    _run([build.hipcc(), f"--offload-arch={build.ARCH}", "-shared", "-fPIC", *HOST_SAN, *objs,
          "-o", lib])
    exe = str(d / "abi_host_check")
    _run([CLANG, *DRIVER_SAN, "-g", "-std=c11", "-I", os.path.join(ROOT, "include"),
          os.path.join(HERE, "abi_host_check.c"), lib, f"-Wl,-rpath,{d}", "-o", exe])
    return exe


def test_abi_host_paths_clean_under_sanitizers(sanitized):
    env = dict(os.environ)
    # the HIP runtime's own allocations are not this library's to check
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sanitized], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{r.stdout}\n{r.stderr[-4000:]}"
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
