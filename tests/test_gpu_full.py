"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: one plan over the whole shape table, every input generated
on the GPU from the benchmark's seeded generators, one muon_step.  Sampled
parameters (every unit of each) are checked against the fp64 oracle: the
orthogonalized update O (read back through update_out), the new weight and
the new momentum; AdamW on sampled rows of the large matrices and on every
vector.  The wide/tall Gram stress set is run with both methods on the same
inputs and their agreement is checked on every unit."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import StepRunner, dev, f64, hp_from, rel, stored
from workloads import configs, gen

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _oracle_hp(d):
    return oracle.OracleHparams(lr=d["lr"], momentum=d["momentum"], weight_decay=d["weight_decay"],
                                nesterov=d["nesterov"], ns_steps=d["ns_steps"], adam_lr=d["adam_lr"],
                                adam_beta1=d["adam_beta1"], adam_beta2=d["adam_beta2"],
                                adam_eps=d["adam_eps"], adam_weight_decay=d["adam_weight_decay"],
                                adam_step=1)


def _inputs(wl, d, wl_id):
    """Parameters, gradients and zero optimizer state, generated on the GPU."""
    P, G, M, EA, ES = [], [], [], [], []
    for p, (kind, dt, rows, cols, _s, _sd) in enumerate(wl.table):
        tdt = gen.torch_dtype(dt)
        P.append(gen.normal(rows, cols, gen.W_STD, gen.stream_seed(0, wl_id, p, 1 << 20), d, tdt))
        if kind == 0:
            G.append(gen.lowrank_gradient(rows, cols, wl.rank, gen.stream_seed(0, wl_id, p, 0), d, tdt))
            M.append(torch.zeros(rows, cols, dtype=torch.float32, device=d))
            EA.append(None)
            ES.append(None)
        else:
            G.append(gen.normal(rows, cols, gen.ADAM_G_STD, gen.stream_seed(0, wl_id, p, 0), d, tdt))
            M.append(None)
            EA.append(torch.zeros(rows, cols, dtype=torch.float32, device=d))
            ES.append(torch.zeros(rows, cols, dtype=torch.float32, device=d))
    return P, G, M, EA, ES


def _check_muon_param(wl, p, W0, G, W1, M1, O, method="standard"):
    """One Muon parameter (all its units) against the oracle run on it alone."""
    row = wl.table[p]
    ref = oracle.muon_step([row], [W0], [G], [np.zeros_like(W0)], [None], [None], _oracle_hp(wl.hp),
                           method=method, want_updates=True)
    worst = 0.0
    for ui, u in enumerate(ref["units"]):
        r0, r1 = u.row0, u.row0 + u.rows
        e = rel(O[r0:r1], ref["O"][ui])
        worst = max(worst, e)
        assert e <= TOL_BF16, (wl.names[p], ui, e)
    dw_ref = stored(ref["W"][0], torch.bfloat16) - W0
    assert rel(W1 - W0, dw_ref) <= TOL_BF16, (wl.names[p], rel(W1 - W0, dw_ref))
    assert rel(M1, ref["M"][0]) <= 1e-6
    return worst


def _run_and_check(wl, wl_id, sample, method=0):
    d = dev()
    print(f"full-size {wl.name}: generating inputs", flush=True)
    P, G, M, EA, ES = _inputs(wl, d, wl_id)
    sel = [wl.names.index(n) for n in sample]
    W0 = {p: f64(P[p]) for p in sel}
    Gh = {p: f64(G[p]) for p in sel}
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) if p in sel else None
            for p, r in enumerate(wl.table)]
    adam = [p for p, r in enumerate(wl.table) if r[0] == 1]
    rows_of = {}
    for p in adam:
        n = wl.table[p][2]
        rows_of[p] = np.unique(np.r_[0:min(n, 32), max(0, n - 32):n])
    A0 = {p: (f64(P[p][rows_of[p]]), f64(G[p][rows_of[p]])) for p in adam}
    print(f"full-size {wl.name}: muon_step over {len(wl.table)} parameters", flush=True)
    StepRunner(wl.table, method=method, device=d).step(P, G, M, EA, ES, hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    worst = 0.0
    for p in sel:
        print(f"  oracle on {wl.names[p]} {wl.table[p][2]}x{wl.table[p][3]}", flush=True)
        worst = max(worst, _check_muon_param(wl, p, W0[p], Gh[p], f64(P[p]), f64(M[p]), f64(outs[p])))
    hp = _oracle_hp(wl.hp)
    for p in adam:
        w0, g = A0[p]
        z = np.zeros_like(w0)
        W, m, v = oracle.adamw_update(w0, g, z, z, 1, hp.adam_lr, hp.adam_beta1, hp.adam_beta2,
                                      hp.adam_eps, hp.adam_weight_decay)
        r = rows_of[p]
        assert rel(f64(EA[p][r]), m) <= 1e-6
        assert rel(f64(ES[p][r]), v) <= 1e-6
        assert rel(f64(P[p][r]) - w0, stored(W, torch.bfloat16) - w0) <= TOL_BF16
    print(f"full-size {wl.name}: worst unit O rel err {worst:.3e}", flush=True)
    del P, G, M, EA, ES, outs
    torch.cuda.empty_cache()


def test_llama3_8b_full_size():
    wl = configs.llama3_8b()
    _run_and_check(wl, 4, ["l0.q", "l7.k", "l31.v", "l12.gate", "l31.down", "l5.up"])


def test_moe_full_size():
    wl = configs.moe_grouped()
    _run_and_check(wl, 5, ["l0.q", "l25.v", "l0.e0.gate", "l13.e7.up", "l25.e63.down"])


def test_wide_gram_both_methods_full_size():
    """32 wide 4096x14336 and 32 tall 14336x4096 units, once with the Gram
    variant and once with the standard method on the same inputs: sampled
    units against the oracle, and the two methods' O on every unit."""
    d = dev()
    wl = configs.wide_gram("gram")
    P, G, M, EA, ES = _inputs(wl, d, 3)
    sample = [0, 31, 32, 63]
    W0 = {p: f64(P[p]) for p in sample}
    Gh = {p: f64(G[p]) for p in sample}
    O = {}
    for method, name in ((1, "gram"), (0, "standard")):
        print(f"full-size wide set, ns_method={name}", flush=True)
        Pm = [p.clone() for p in P]
        Mm = [m.clone() for m in M]
        outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) for r in wl.table]
        StepRunner(wl.table, method=method, device=d).step(Pm, G, Mm, EA, ES, hp_from(wl.hp),
                                                           update_outs=outs)
        torch.cuda.synchronize()
        for p in sample:
            print(f"  oracle on {wl.names[p]} ({name})", flush=True)
            _check_muon_param(wl, p, W0[p], Gh[p], f64(Pm[p]), f64(Mm[p]), f64(outs[p]))
        O[name] = outs
        del Pm, Mm
    agree = max(float((a - b).norm() / b.norm()) for a, b in zip(O["gram"], O["standard"]))
    print(f"full-size wide set: max over units of |O_gram - O_std| / |O_std| = {agree:.3e}", flush=True)
    assert agree <= 2 * TOL_BF16
    del P, G, M, O
    torch.cuda.empty_cache()
