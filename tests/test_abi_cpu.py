"""Host-side checks of libmuon that need no GPU: the library loads and
exports every function include/libmuon.h declares, the planner matches the
oracle's independent brute-force bucketing bit for bit, and invalid
arguments are rejected before any HIP call."""
import ctypes
import os
import re

import pytest

import oracle
from oracle import cref
from workloads import configs

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    try:
        return mo.lib()
    except RuntimeError as e:  # not built in this checkout
        pytest.skip(str(e))


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.append(m.group(1))
    return names


def test_exports_every_declared_function():
    L = _lib_or_skip()
    names = declared_functions()
    assert set(names) >= {"muon_step", "ns_orthogonalize", "muon_plan_create"}
    for n in names:
        assert hasattr(L, n), f"libmuon.so does not export {n}"
    assert sorted(names) == sorted(mo.EXPORTED)
    assert mo.muon_version() >= 100
    for code in range(-8, 1):
        assert mo.muon_status_string(code) != "unknown status"


@pytest.mark.parametrize("name", list(configs.ALL))
@pytest.mark.parametrize("ns_dtype", [-1, 0])
@pytest.mark.parametrize("auto", [False, True])
def test_plan_matches_oracle_bit_exact(name, ns_dtype, auto):
    _lib_or_skip()
    wl = configs.ALL[name]()
    method = 2 if auto else (1 if wl.method == "gram" else 0)
    plan = mo.muon_plan_create(wl.table, method, ns_dtype)
    units, keys, members = oracle.plan_buckets(wl.table, method, ns_dtype)
    got_b = mo.muon_plan_buckets(plan)
    exp_b, first = [], 0
    for k, mem in zip(keys, members):
        exp_b.append(tuple(k) + (first, len(mem)))
        first += len(mem)
    assert got_b == exp_b
    exp_u = []
    for mem in members:
        for ui in mem:
            u = units[ui]
            exp_u.append((u.param, u.row0, u.rows, u.cols, int(u.tall),
                          u.scale_dim if u.scale_dim > 0 else max(u.rows, u.cols)))
    assert mo.muon_plan_units(plan) == exp_u
    # the C++ reference's planner, written separately, agrees bit for bit
    c_units, c_buckets = cref.plan(wl.table, method, ns_dtype)
    assert c_buckets == exp_b
    assert c_units == exp_u
    ws = mo.muon_plan_workspace_bytes(plan)
    assert ws > 0


def test_plan_mixed_and_edge_tables():
    _lib_or_skip()
    table = [(0, 1, 6, 4, 2, 0),      # 3 row blocks 2x4
             (1, 1, 1, 7, 0, 0),      # vector -> AdamW
             (0, 0, 5, 3, 0, 11),     # tall fp32 with a scale override
             (0, 1, 0, 9, 0, 0),      # empty: no unit
             (0, 1, 2, 4, 0, 0),      # same bucket as the blocks
             (0, 0, 37, 50, 0, 0)]    # ragged
    plan = mo.muon_plan_create(table)
    units, keys, members = oracle.plan_buckets(table, 0)
    assert [b[:6] for b in mo.muon_plan_buckets(plan)] == [tuple(k) for k in keys]
    assert [b[7] for b in mo.muon_plan_buckets(plan)] == [len(m) for m in members]
    assert mo.muon_plan_units(plan)[3] == (4, 0, 2, 4, 0, 4)
    empty = mo.muon_plan_create([])
    assert mo.muon_plan_buckets(empty) == [] and mo.muon_plan_workspace_bytes(empty) == 0


@pytest.mark.parametrize("row,status", [
    ((2, 1, 4, 4, 0, 0), -1),    # unknown kind
    ((0, 5, 4, 4, 0, 0), -3),    # unknown dtype
    ((0, 1, -1, 4, 0, 0), -2),   # negative rows
    ((0, 1, 6, 4, 4, 0), -2),    # split does not divide rows
    ((1, 1, 6, 4, 2, 0), -2),    # split on an AdamW row
    ((0, 1, 4, 1 << 31, 0, 0), -2),  # side too large
])
def test_plan_rejects(row, status):
    _lib_or_skip()
    with pytest.raises(mo.MuonError) as e:
        mo.muon_plan_create([row])
    assert e.value.status == status
    with pytest.raises(mo.MuonError) as e:
        mo.muon_plan_create([(0, 1, 4, 4, 0, 0)], ns_method=7)
    assert e.value.status == -4


def test_auto_method_resolution():
    _lib_or_skip()
    # Gram only where its fp16 chain is accurate, m >= 512 and n >= 3m; the
    # plan reports the resolved method
    table = [(0, 1, 4096, 14336, 0, 0), (0, 1, 14336, 4096, 0, 0), (0, 1, 4096, 4096, 0, 0),
             (0, 1, 1024, 4096, 0, 0), (0, 1, 256, 4096, 0, 0), (0, 1, 600, 1799, 0, 0),
             (0, 1, 600, 1800, 0, 0), (0, 1, 511, 4096, 0, 0), (0, 1, 512, 1536, 0, 0)]
    got = [b[5] for b in mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_AUTO))]
    assert got == [1, 1, 0, 1, 0, 0, 1, 0, 1]
    # auto never changes the compute dtype
    assert all(b[4] == 1 for b in mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_AUTO)))


def test_restarted_gram_resolution():
    """The restarted Gram chain keeps the 16-bit compute dtype for m >= 256
    at any aspect ratio (the restart holds the fp16 chain within tolerance);
    a smaller unit, and any fp32 request, is taken as a plain Gram request;
    its workspace holds one more n x m copy."""
    _lib_or_skip()
    table = [(0, 1, 256, 1024, 0, 0), (0, 1, 768, 768, 0, 0), (0, 1, 768, 3072, 0, 0),
             (0, 1, 255, 300, 0, 0), (0, 1, 64, 200, 0, 0), (0, 0, 256, 512, 0, 0), (0, 0, 512, 1536, 0, 0)]
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_GRAM_RESTART))
    assert [x[5] for x in b] == [3, 3, 3, 1, 1, 0, 1]
    assert [x[4] for x in b] == [1, 1, 1, 0, 0, 0, 0]
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_GRAM_RESTART, 1))
    assert [x[5] for x in b] == [3, 3, 3, 1, 1, 3, 3] and [x[4] for x in b] == [1, 1, 1, 0, 0, 1, 1]
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_GRAM_RESTART, 0))
    assert [x[5] for x in b] == [0, 0, 1, 0, 0, 0, 1] and [x[4] for x in b] == [0] * 7
    for shape in ((256, 1024), (768, 768), (3072, 768)):
        r = mo.ns_orthogonalize_workspace_bytes(*shape, 1, mo.MUON_NS_GRAM_RESTART)
        g = mo.ns_orthogonalize_workspace_bytes(*shape, 1, mo.MUON_NS_GRAM)
        if min(shape) >= 512 and max(shape) >= 3 * min(shape):
            # Gram in fp16 too: exactly one more n x mp 16-bit copy (with the
            # layout's alignment slack)
            extra = max(shape) * ((min(shape) + 7) // 8 * 8) * 2
            assert extra <= r - g <= extra + 256
        else:
            assert r > 0
    assert (mo.ns_orthogonalize_workspace_bytes(256, 1024, 0, mo.MUON_NS_GRAM_RESTART)
            == mo.ns_orthogonalize_workspace_bytes(256, 1024, 0, mo.MUON_NS_STANDARD))


def test_explicit_gram_outside_fp16_region():
    """An explicit Gram request outside m >= 512, n >= 3m: a bf16 unit runs
    the Gram chain in fp32 (compute dtype 0), an fp32 unit the standard
    method; inside the region Gram runs in the requested dtype."""
    _lib_or_skip()
    table = [(0, 1, 256, 1024, 0, 0), (0, 1, 768, 768, 0, 0), (0, 1, 768, 3072, 0, 0),
             (0, 1, 3072, 768, 0, 0), (0, 1, 512, 860, 0, 0), (0, 0, 256, 512, 0, 0),
             (0, 0, 512, 1536, 0, 0)]
    meth = lambda b: [x[5] for x in b]
    cdt = lambda b: [x[4] for x in b]
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_GRAM))
    assert meth(b) == [1, 1, 1, 1, 1, 0, 1]
    assert cdt(b) == [0, 0, 1, 1, 0, 0, 0]
    # compute forced to bf16: every unit runs Gram, outside the region in fp32
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_GRAM, 1))
    assert meth(b) == [1] * 7
    assert cdt(b) == [0, 0, 1, 1, 0, 0, 1]
    # compute forced to fp32: Gram only inside the region
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_GRAM, 0))
    assert meth(b) == [0, 0, 1, 1, 0, 0, 1]
    assert cdt(b) == [0] * 7
    # the standard method keeps the requested dtype
    b = mo.muon_plan_buckets(mo.muon_plan_create(table, mo.MUON_NS_STANDARD))
    assert meth(b) == [0] * 7 and cdt(b) == [1, 1, 1, 1, 1, 0, 0]
    # ns_orthogonalize sizes its workspace for the same resolution: an fp32
    # Gram request outside the region takes the standard method's workspace,
    # a bf16 one fp32 working copies (more than its standard workspace)
    assert (mo.ns_orthogonalize_workspace_bytes(256, 1024, 0, mo.MUON_NS_GRAM)
            == mo.ns_orthogonalize_workspace_bytes(256, 1024, 0, mo.MUON_NS_STANDARD))
    assert (mo.ns_orthogonalize_workspace_bytes(256, 1024, 1, mo.MUON_NS_GRAM)
            > mo.ns_orthogonalize_workspace_bytes(256, 1024, 1, mo.MUON_NS_STANDARD))


def test_step_validation_before_any_launch():
    L = _lib_or_skip()
    from matrix_orthogonalizing_optimizer_amd import _lib as B
    plan = mo.muon_plan_create([(0, 1, 4, 8, 0, 0)])
    hp = mo.make_hparams()
    ptrs = (B.MuonParamPtrs * 1)()
    ptrs[0] = B.MuonParamPtrs(0x1000, 0x2000, 0x3000, None, None, None)
    ws = mo.muon_plan_workspace_bytes(plan)
    # table size mismatch
    assert L.muon_step(plan.handle, ptrs, 2, ctypes.byref(hp), 0x10000, ws, None) == -7
    # null plan / hparams / pointer arrays
    assert L.muon_step(None, ptrs, 1, ctypes.byref(hp), 0x10000, ws, None) == -1
    assert L.muon_step(plan.handle, ptrs, 1, None, 0x10000, ws, None) == -1
    assert L.muon_step(plan.handle, None, 1, ctypes.byref(hp), 0x10000, ws, None) == -1
    # workspace too small / missing
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(hp), 0x10000, ws - 1, None) == -5
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(hp), None, ws, None) == -5
    # misaligned bf16 param, missing momentum
    ptrs[0] = B.MuonParamPtrs(0x1001, 0x2000, 0x3000, None, None, None)
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(hp), 0x10000, ws, None) == -1
    ptrs[0] = B.MuonParamPtrs(0x1000, 0x2000, None, None, None, None)
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(hp), 0x10000, ws, None) == -1
    # non-finite hyperparameter, bad step count, non-finite coefficient
    ptrs[0] = B.MuonParamPtrs(0x1000, 0x2000, 0x3000, None, None, None)
    bad = mo.make_hparams(lr=float("nan"))
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(bad), 0x10000, ws, None) == -1
    bad = mo.make_hparams(ns_steps=0)
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(bad), 0x10000, ws, None) == -1
    # (the binding refuses a non-finite coefficient itself: pass the array raw)
    bad = mo.make_hparams(ns_steps=2)
    raw = (ctypes.c_float * 6)(1.0, float("inf"), 0.0, 1.0, 0.0, 0.0)
    bad.coeffs = ctypes.cast(raw, ctypes.POINTER(ctypes.c_float))
    assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(bad), 0x10000, ws, None) == -1
    # unknown scale mode, negative or non-finite extra scale
    for bad in (mo.make_hparams(scale_mode=3), mo.make_hparams(extra_scale=-1.0),
                mo.make_hparams(extra_scale=float("inf"))):
        assert L.muon_step(plan.handle, ptrs, 1, ctypes.byref(bad), 0x10000, ws, None) == -1


def test_ns_orthogonalize_validation():
    L = _lib_or_skip()
    assert mo.ns_orthogonalize_workspace_bytes(0, 5, 1) == 0
    nb = mo.ns_orthogonalize_workspace_bytes(64, 96, 1)
    assert nb > 64 * 96 * 2 * 2
    assert mo.ns_orthogonalize_workspace_bytes(96, 64, 1) == nb  # tall uses the same shape
    f = L.ns_orthogonalize
    assert f(0x1000, 64, 96, 96, 9, 5, None, 0, 0x10000, nb, None) == -3
    assert f(0x1000, 64, 96, 96, 1, 5, None, 4, 0x10000, nb, None) == -4
    assert f(0x1000, 64, 96, 96, 1, 5, None, -1, 0x10000, nb, None) == -4
    # the restarted Gram chain needs more than the standard workspace
    assert f(0x1000, 64, 96, 96, 1, 5, None, 3, 0x10000, nb, None) == -5
    assert f(0x1000, 64, 96, 90, 1, 5, None, 0, 0x10000, nb, None) == -2
    assert f(0x1000, 64, 96, 96, 1, 0, None, 0, 0x10000, nb, None) == -1
    assert f(None, 64, 96, 96, 1, 5, None, 0, 0x10000, nb, None) == -1
    assert f(0x1000, 64, 96, 96, 1, 5, None, 0, 0x10000, nb - 1, None) == -5
    assert f(0x1000, 0, 96, 96, 1, 5, None, 0, None, 0, None) == 0   # empty: nothing to do


def test_probe_validation():
    L = _lib_or_skip()
    import ctypes as C
    fl = C.c_double()
    assert L.muon_probe_mfma(0, 10, 0x1000, C.byref(fl), None) == -1
    assert L.muon_probe_mfma(4, 0, 0x1000, C.byref(fl), None) == -1
    assert L.muon_probe_mfma(4, 10, None, C.byref(fl), None) == -1
    assert L.muon_probe_mfma(4, 10, 0x1000, None, None) == -1
    assert L.muon_probe_copy(0x1000, 0x2000, 0, None) == -1      # nothing to copy
    assert L.muon_probe_copy(0x1000, 0x2000, 24, None) == -1     # not a multiple of 16
    assert L.muon_probe_copy(0x1008, 0x2000, 32, None) == -1     # misaligned source
    assert L.muon_probe_copy(0x1000, 0x2004, 32, None) == -1     # misaligned destination
    assert L.muon_probe_copy(None, 0x2000, 32, None) == -1


def test_step_binding_checks_buffers():
    """The Python binding refuses tensors that do not match the table (no
    launch happens: the check precedes the library call)."""
    _lib_or_skip()
    import torch
    plan = mo.muon_plan_create([(0, 1, 4, 8, 0, 0), (1, 0, 1, 8, 0, 0)])
    hp = mo.make_hparams()
    ok = [torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(1, 8, dtype=torch.float32)]
    moms = [torch.zeros(4, 8), None]
    ea = [None, torch.zeros(1, 8)]
    es = [None, torch.zeros(1, 8)]
    bad_cases = [
        ([torch.zeros(4, 8, dtype=torch.float32), ok[1]], ok, moms),          # param dtype
        ([torch.zeros(4, 9, dtype=torch.bfloat16), ok[1]], ok, moms),         # param shape
        (ok, [torch.zeros(8, 4, dtype=torch.bfloat16).t(), ok[1]], moms),     # not contiguous
        (ok, ok, [torch.zeros(4, 8, dtype=torch.bfloat16), None]),            # momentum dtype
        (ok[:1], ok, moms),                                                   # list length
    ]
    for p, g, m in bad_cases:
        with pytest.raises(ValueError):
            mo.muon_step(plan, p, g, m, ea, es, hp, 0x10000)


@pytest.mark.parametrize("coeffs,steps", [
    ([(3.4445, -4.775, 2.0315)] * 3, 5),   # too few rows
    ([(3.4445, -4.775, 2.0315)] * 6, 5),   # too many rows
    ([(3.4445, -4.775)] * 5, 5),           # rows of two
    ([(1.0, float("nan"), 0.0)] * 2, 2),   # non-finite
])
def test_binding_rejects_bad_coefficient_tables(coeffs, steps):
    """A coefficient table must have exactly `steps` rows of three finite
    numbers (or be a single triple): the library reads 3 * steps floats."""
    with pytest.raises(ValueError):
        mo.make_hparams(ns_steps=steps, coeffs=coeffs)
    import torch
    with pytest.raises(ValueError):
        mo.ns_orthogonalize(torch.zeros(4, 8), steps=steps, coeffs=coeffs)
    # one triple is broadcast to every step
    hp = mo.make_hparams(ns_steps=steps, coeffs=(3.4445, -4.775, 2.0315))
    assert [hp.coeffs[i] for i in range(3 * steps)] == pytest.approx([3.4445, -4.775, 2.0315] * steps)


def test_binding_rejects_host_tensors():
    """Tensors in host memory never reach the library as device pointers:
    the binding raises before any call (no GPU is touched)."""
    _lib_or_skip()
    import torch
    X = torch.zeros(64, 96, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device memory"):
        mo.ns_orthogonalize(X)
    plan = mo.muon_plan_create([(0, 1, 4, 8, 0, 0)])
    hp = mo.make_hparams()
    p = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device memory"):
        mo.muon_step(plan, [p], [p.clone()], [torch.zeros(4, 8)], [None], [None], hp,
                     torch.empty(mo.muon_plan_workspace_bytes(plan), dtype=torch.uint8))
    host = torch.zeros(1 << 12, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device memory"):
        mo.muon_probe_copy(host, host.clone(), 1 << 12)
    with pytest.raises(ValueError, match="device memory"):
        mo.muon_probe_copy_lds(host, host.clone(), 1 << 12)
    with pytest.raises(ValueError, match="device memory"):
        mo.muon_probe_mfma(4, 8, torch.zeros(4))


def _random_table(rng, n):
    rows = []
    for _ in range(n):
        kind = int(rng.integers(0, 2))
        dt = int(rng.integers(0, 2))
        if kind == 1:
            rows.append((1, dt, int(rng.choice([1, 3, 64])), int(rng.integers(0, 300)), 0, 0))
            continue
        shape = [int(rng.choice([0, 1, 7, 64, 128, 300, 512, 600, 1536, 1800, 2048])) for _ in range(2)]
        split = 0
        if shape[0] > 0 and rng.random() < 0.3:
            divs = [h for h in (1, 2, 3, 4, 64, 128, 256) if shape[0] % h == 0]
            split = int(rng.choice(divs))
        sd = int(rng.choice([0, 0, 0, 11, 4096]))
        rows.append((0, dt, shape[0], shape[1], split, sd))
    return rows


@pytest.mark.parametrize("seed", range(40))
def test_plan_random_tables_match_both_references(seed):
    """Random shape tables (empty, tiny, ragged, split, tall, wide, repeated
    shapes; every method and compute-dtype option): the library's plan equals
    both references' independent planners bit for bit."""
    _lib_or_skip()
    import numpy as np
    rng = np.random.default_rng(1000 + seed)
    table = _random_table(rng, int(rng.integers(1, 25)))
    for method in (0, 1, 2, 3):
        for ns_dtype in (-1, 0, 1):
            plan = mo.muon_plan_create(table, method, ns_dtype)
            units, keys, members = oracle.plan_buckets(table, method, ns_dtype)
            exp_b, first = [], 0
            for k, mem in zip(keys, members):
                exp_b.append(tuple(k) + (first, len(mem)))
                first += len(mem)
            exp_u = [(units[ui].param, units[ui].row0, units[ui].rows, units[ui].cols, int(units[ui].tall),
                      units[ui].scale_dim if units[ui].scale_dim > 0 else max(units[ui].rows, units[ui].cols))
                     for mem in members for ui in mem]
            assert mo.muon_plan_buckets(plan) == exp_b, (seed, method, ns_dtype)
            assert mo.muon_plan_units(plan) == exp_u, (seed, method, ns_dtype)
            c_units, c_buckets = cref.plan(table, method, ns_dtype)
            assert c_buckets == exp_b and c_units == exp_u, (seed, method, ns_dtype)
            has_work = bool(exp_u) or any(r[0] == 1 for r in table)
            assert (mo.muon_plan_workspace_bytes(plan) > 0) == has_work
