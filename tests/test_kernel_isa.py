"""Static properties of the gfx950 code the kernel sources compile to (host
only: hipcc emits the device assembly, nothing runs on a GPU).

  * No kernel uses flat memory instructions: every operand lives in global
    memory or LDS, and a flat load also counts against the LDS wait counter,
    so a wait for LDS before a barrier would wait for the global loads as
    well (the stream-K kernel once lost the global address space that way).
  * No kernel spills to scratch memory.
  * The MFMA kernels stay within the registers that the split's plans
    assume: four workgroups of the 64 x 64 tile with two register sets per
    CU, three with four sets, one of each 8-wave tile (the stream-K kernel:
    three of either 64 x 64 tile).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from tiling_roofline_analysis_amd import build


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [build.hipcc(), *build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    with open(out) as fh:
        return fh.read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("isa"))
    srcs = [s for s in build.SOURCES if s != "tra_gemm.hip"]
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, d), srcs))
    return dict(zip(srcs, texts))


def _kernels(text: str):
    """(name, vgprs, scratch bytes) of every kernel in the metadata."""
    names = re.findall(r"^\s+\.name:\s+(\S+)", text, re.M)
    vgprs = [int(x) for x in re.findall(r"^\s+\.vgpr_count:\s+(\d+)", text, re.M)]
    scratch = [int(x) for x in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", text,
                                          re.M)]
    assert len(names) == len(vgprs) == len(scratch) and names
    return list(zip(names, vgprs, scratch))


def test_no_flat_memory_instructions(asm):
    for src, text in asm.items():
        code = "\n".join(line.split(";")[0] for line in text.splitlines())
        assert not re.search(r"^\s+flat_", code, re.M), f"{src} uses flat memory instructions"


def test_no_scratch(asm):
    for src, text in asm.items():
        for name, _, scratch in _kernels(text):
            assert scratch == 0, f"{name} ({src}) spills {scratch} bytes to scratch"


# tile (BM, BN, BK, WM, WN, NR) -> largest VGPR count that still gives the
# planned workgroups per CU (512 VGPRs per SIMD lane; 4 waves per workgroup
# on the 64 x 64 tile, 8 on the others)
VGPR_BUDGET = {
    "64ELi64ELi16ELi32ELi32ELi2": 128,    # four workgroups a CU
    "64ELi64ELi16ELi32ELi32ELi4": 168,    # three
    "128ELi128ELi16ELi64ELi32ELi2": 256,  # one
    "256ELi128ELi16ELi64ELi64ELi4": 256,  # one
}


def test_mfma_register_budgets(asm):
    seen = set()
    for name, vgprs, _ in _kernels(asm["gemm_mfma.hip"]):
        if "gemm_mfma_f32_fixup" in name:
            continue
        for key, budget in VGPR_BUDGET.items():
            if f"MfmaTileILi{key}E" in name:
                seen.add(key)
                if "gemm_mfma_f32_sk" in name:
                    budget = max(budget, 168)    # planned at three a CU
                assert vgprs <= budget, f"{name}: {vgprs} VGPRs, plan assumes <= {budget}"
    assert seen == set(VGPR_BUDGET)


def _functions(text: str):
    """name -> assembly body of every kernel function."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):\s*;\s*@\1\n(.*?)^\s+s_endpgm", text, re.M | re.S):
        out.setdefault(m.group(1), m.group(2))
    return out


def _loops(body: str):
    """The instruction text of each loop: from a loop header label to the
    branch back to it."""
    loops = []
    for m in re.finditer(r"^(\.LBB\w+):[^\n]*Loop Header", body, re.M):
        label = m.group(1)
        end = re.search(rf"^\s+s_cbranch\w*\s+{re.escape(label)}\s*$", body[m.end():], re.M)
        if end:
            loops.append(body[m.end():m.end() + end.end()])
    return loops


def _whole_functions(text: str):
    """name -> assembly of every kernel function, up to its end label."""
    return {m.group(1): m.group(2) for m in
            re.finditer(r"^(_Z\S+):\s*;\s*@\1\n(.*?)^\.Lfunc_end", text, re.M | re.S)}


def _direct_load_kernels(text: str):
    return {n: b for n, b in _whole_functions(text).items()
            if n.startswith("_ZN3tra12_GLOBAL__N_113gemm_mfma_f32INS0_8MfmaTile")
            and re.search(r"Lb1ELi[12]EEEvlllPKflS5_lPflNS0_6SkPlanEiii$", n)}


def test_direct_load_fragment_reads_wait_only_at_barriers(asm):
    # Every wait for direct loads in these kernels is an explicit
    # s_waitcnt vmcnt(n) lgkmcnt(0) followed by s_barrier.  A vector-memory
    # wait that lands right in front of an LDS read is one the compiler put
    # there because it could not tell the read's stage from a stage still
    # being loaded; it waits for every load in flight.  (A loop over the
    # last slices of a tile with run-time conditions got one before each
    # fragment read.)
    funcs = _direct_load_kernels(asm["gemm_mfma.hip"])
    assert len(funcs) == 2, sorted(funcs)
    mem = re.compile(r"(ds_|global_|buffer_|s_barrier|s_endpgm)")
    for name, body in funcs.items():
        lines = [x.split(";")[0].strip() for x in body.splitlines()]
        lines = [x for x in lines if x and not x.endswith(":")]
        waits = 0
        for i, x in enumerate(lines):
            if not (x.startswith("s_waitcnt") and "vmcnt" in x):
                continue
            nxt = next((y for y in lines[i + 1:] if mem.match(y)), "")
            assert not nxt.startswith("ds_read"), f"{name}: '{x}' right before '{nxt}'"
            waits += nxt == "s_barrier"
        assert waits >= 8, f"{name}: {waits} explicit waits"


def test_direct_load_loops_keep_loads_in_flight(asm):
    # The direct-load kernels (gemm_mfma_f32<T, true, 1 or 2>) stage slices
    # with buffer_load_dwordx4 ... lds and wait for them with explicit
    # counts.  Their main loop must not wait for every load in flight
    # (vmcnt(0)): that is what the compiler inserts before an LDS read that
    # may alias an earlier direct load, and it would serialise the pipeline.
    # It must not compute vector addresses either: each slice moves only the
    # buffer's uniform base (scalar adds), since 64-bit vector adds beside
    # the MFMAs cost 6% at 1024^3.
    funcs = {n: b for n, b in _functions(asm["gemm_mfma.hip"]).items()
             if n.startswith("_ZN3tra12_GLOBAL__N_113gemm_mfma_f32INS0_8MfmaTile")
             and re.search(r"Lb1ELi[12]EEEvlllPKflS5_lPflNS0_6SkPlanEiii$", n)}
    # the 64 x 64 tile (both 64 x 64 classes launch it), with full slices
    # and with a slice past K
    assert len(funcs) == 2, sorted(funcs)
    dma = re.compile(r"^\s+buffer_load_dwordx4 .* lds\s*$", re.M)
    for name, body in funcs.items():
        code = "\n".join(line.split(";")[0] for line in body.splitlines())
        assert dma.search(code), name
        # every direct load writes LDS at the address in M0, so the kernel
        # sets M0 (a compiler of this family has been seen to drop that for
        # a direct load into an LDS array at a constant address)
        assert re.search(r"^\s+s_\w+\s+m0,", code, re.M), f"{name}: M0 never set"
        main = [lp for lp in _loops(body)
                if dma.search("\n".join(x.split(";")[0] for x in lp.splitlines()))
                and "v_mfma_f32_32x32x2_f32" in lp]
        assert main, f"{name}: no loop with direct loads and MFMAs"
        lp = "\n".join(line.split(";")[0] for line in main[0].splitlines())
        assert "vmcnt(0)" not in lp, f"{name}: main loop waits for every load in flight"
        assert re.search(r"s_waitcnt vmcnt\([1-9]\d*\) lgkmcnt\(0\)", lp), name
        valu = [x.strip() for x in lp.splitlines()
                if re.match(r"\s+v_", x) and not re.match(r"\s+v_mfma", x)]
        assert len(valu) <= 2, f"{name}: vector work in the main loop: {valu}"
