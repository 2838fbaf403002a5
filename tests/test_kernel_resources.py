"""Compiled-code checks of the HIP kernels (no GPU needed: hipcc
cross-compiles for gfx950).

- No kernel uses scratch memory: a spill or a stack array in these kernels
  (for example the GEMM accumulators indexed with a run-time value) costs a
  large part of their time, and nothing else would reveal it.
- No buffer load or store of the GEMM (direct-to-LDS operand copies, the
  epilogue's loads of the addend and of the old parameter values, its
  stores) sits in a waterfall loop: they take a scalar buffer resource, and
  if the compiler cannot prove its operands uniform it loops over the
  distinct values lane by lane.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from matrix_orthogonalizing_optimizer_amd import build as B

SOURCES = ["gemm_bf16.hip", "gemm_f16.hip", "gemm_f32.hip", "kernels_elem.hip"]


def _hipcc_or_skip():
    h = B._hipcc()
    if not (os.path.exists(h) or shutil.which(h)):
        pytest.skip("hipcc not available")
    return h


def _compile(src, extra):
    cmd = [_hipcc_or_skip()] + B.hip_flags() + ["--cuda-device-only"] + extra + [os.path.join(B.CSRC, src)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r


@pytest.fixture(scope="module")
def resource_reports(tmp_path_factory):
    d = tmp_path_factory.mktemp("res")

    def one(src):
        r = _compile(src, ["-c", "-o", str(d / (src + ".o")), "-Rpass-analysis=kernel-resource-usage"])
        names = re.findall(r"Function Name: (\S+)", r.stderr)
        scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
        assert len(names) == len(scratch) and names, src
        return src, list(zip(names, scratch))

    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(one, SOURCES))


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(resource_reports, src):
    bad = [(n, s) for n, s in resource_reports[src] if s != 0]
    assert not bad, f"kernels with scratch memory in {src}: {bad}"


@pytest.mark.parametrize("src", ["gemm_bf16.hip", "gemm_f16.hip", "gemm_f32.hip"])
def test_buffer_accesses_not_in_waterfall_loops(tmp_path, src):
    out = tmp_path / (src + ".s")
    _compile(src, ["-S", "-o", str(out)])
    lines = [l.strip() for l in out.read_text().splitlines()]
    copies = [i for i, l in enumerate(lines) if l.startswith("buffer_load_dword") and l.endswith(" lds")]
    assert copies, "no direct-to-LDS copies found"
    accesses = [i for i, l in enumerate(lines) if l.startswith(("buffer_load_dword", "buffer_store_dword"))]
    assert len(accesses) > len(copies), "no epilogue buffer accesses found"
    for i in accesses:
        window = lines[max(0, i - 4):i]
        assert not any(w.startswith("s_and_saveexec") for w in window), \
            f"{src}: buffer access at line {i} is inside a waterfall loop: {window + [lines[i]]}"


@pytest.mark.parametrize("src", ["gemm_bf16.hip", "gemm_f16.hip", "gemm_f32.hip"])
def test_gemm_kernels_use_no_flat_memory_instructions(tmp_path, src):
    """Every global access of the GEMM kernels is a buffer or global
    instruction: a FLAT access also counts in lgkmcnt, so the epilogue's
    next LDS wait would wait for that global store to complete."""
    out = tmp_path / (src + ".s")
    _compile(src, ["-S", "-o", str(out)])
    flat = [l.strip() for l in out.read_text().splitlines() if l.strip().startswith("flat_")]
    assert not flat, f"{src}: {len(flat)} FLAT instructions, e.g. {flat[:3]}"
