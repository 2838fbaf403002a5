"""The C ABI used from plain C: tests/c/abi_check.c is compiled as C99 with
-pedantic -Werror against include/libmuon.h, linked against the in-tree
libmuon.so and run (host calls only, no GPU).  Its plan output is compared
with the numpy reference's planner."""
import os
import shutil
import subprocess

import pytest

import oracle

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_uses_the_abi(tmp_path):
    try:
        mo.lib()
    except RuntimeError as e:
        pytest.skip(str(e))
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        pytest.skip("no C compiler")
    pkg = os.path.join(ROOT, "matrix_orthogonalizing_optimizer_amd")
    exe = str(tmp_path / "abi_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", pkg, "-lmuon",
                    f"-Wl,-rpath,{pkg}", "-o", exe], check=True)
    r = subprocess.run([exe], stdout=subprocess.PIPE, text=True)
    assert r.returncode == 0, (r.returncode, r.stdout)
    lines = r.stdout.splitlines()
    table = [(0, 1, 2304, 768, 768, 0), (0, 1, 3072, 768, 0, 0), (0, 0, 300, 701, 0, 0), (1, 1, 1, 768, 0, 0)]
    units, keys, members = oracle.plan_buckets(table, 0)
    exp_b, first = [], 0
    for k, mem in zip(keys, members):
        exp_b.append("bucket " + " ".join(str(x) for x in tuple(k) + (first, len(mem))))
        first += len(mem)
    exp_u = ["unit " + " ".join(str(x) for x in (units[i].param, units[i].row0, units[i].rows, units[i].cols,
                                                   int(units[i].tall), max(units[i].rows, units[i].cols)))
             for mem in members for i in mem]
    assert [l for l in lines if l.startswith("bucket")] == exp_b
    assert [l for l in lines if l.startswith("unit")] == exp_u
    assert "workspace_nonzero 1" in lines
    assert "hybrid_last 1.8750 -1.2500 0.3750" in lines
    assert "ns_workspace_fits_noalloc 1" in lines
    assert "status workspace missing or too small" in lines
    assert "version_ok 1" in lines
