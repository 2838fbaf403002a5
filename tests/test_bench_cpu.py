"""CPU checks of the benchmark's bookkeeping (no GPU): the FLOP counts its
TFLOP/s figures divide, the unit shapes, the committed counter summary it
reports traffic from, and the single-GPU guard.

- the nominal Newton-Schulz count of the 8B-shaped set is the 665.9 TFLOP per
  five-step step of the design notes, summed here from the layer shapes;
- executed_flops equals a brute-force count of the output tiles each GEMM
  kind computes (every upper-triangle tile of a symmetric product, every
  tile of the others), for every workload's plan and both methods;
- the update GEMM's traffic figure is present: the committed counters were
  taken from the GEMM sources as they are now;
- more than one GPU is refused with a message, before any GPU work.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_nominal_ns_flops_of_the_8b_set():
    layer = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (4096, 14336), (4096, 14336), (4096, 14336)]
    per_step = 32 * sum(4 * m * m * n + 2 * m ** 3 for m, n in layer)
    wl = configs.llama3_8b()
    assert configs.ns_flops(wl.table) == per_step
    assert round(5 * per_step / 1e12, 1) == 665.9


@pytest.mark.parametrize("name", sorted(configs.ALL))
def test_unit_shapes_match_the_plan(name):
    mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")
    b = _bench()
    wl = configs.ALL[name]()
    plan = mo.muon_plan_create(wl.table, 0)
    units = mo.muon_plan_units(plan)
    assert sorted(b.unit_shapes(wl.table)) == sorted((min(r, c), max(r, c)) for _p, _r0, r, c, _t, _sd in units)


def _brute_executed(buckets, steps):
    out = {}

    def add(k, v):
        out[k] = out.get(k, 0.0) + v

    for m, n, _tall, _pdt, _cdt, method, _first, count in buckets:
        T = 256 if m > 192 else 128
        tm = -(-m // T)
        tn = -(-n // T)
        upper = sum(1 for i in range(tm) for j in range(tm) if j >= i)
        full = tm * tn
        tile = 2.0 * T * T
        if method == 0:
            add("ns_gram_A", steps * count * upper * tile * n)
            add("ns_poly_P", steps * count * upper * tile * m)
            if steps > 1:
                add("ns_update_PX", (steps - 1) * count * full * tile * m)
            add("ns_final_update", count * full * tile * m)
        else:
            # walk the launch sequence of the Gram chain step by step
            ra = (steps + 1) // 2 if method == 3 and steps >= 2 else 0
            add("gram_r0", count * upper * tile * n)
            have_q = False
            for k in range(steps):
                last = k == steps - 1
                add("gram_p", count * upper * tile * m)
                if have_q:
                    add("gram_q", count * upper * tile * m)
                have_q = True
                if not last and ra and k + 1 == ra:
                    add("ns_update_PX", count * full * tile * m)
                    add("gram_r0", count * upper * tile * n)
                    have_q = False
                elif not last:
                    add("gram_t", count * upper * tile * m)
                    add("gram_r", count * upper * tile * m)
            add("ns_final_update", count * full * tile * m)
    return out


@pytest.mark.parametrize("name", sorted(configs.ALL))
@pytest.mark.parametrize("method", [0, 1, 2, 3])
def test_executed_flops_brute_force(name, method):
    mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")
    b = _bench()
    wl = configs.ALL[name]()
    buckets = mo.muon_plan_buckets(mo.muon_plan_create(wl.table, method))
    for steps in (1, 2, 5, 10):
        assert b.executed_flops(buckets, steps) == _brute_executed(buckets, steps)


def test_committed_update_gemm_counters_match_the_sources():
    b = _bench()
    t = b.measured_traffic("llama3_8b_bf16")
    assert t is not None, "GEMM sources changed since profiles/llama3_8b_bf16_update_gemm_hbm_counters.md was taken"
    assert 8.36e9 < t < 5e10  # at least the algorithmic bytes of a launch


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
