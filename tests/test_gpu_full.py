"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: one plan over the whole shape table, every input generated
on the GPU from the benchmark's seeded generators, one muon_step.

Checked against the fp64 numpy reference (BLAS matmul; the plain C++ one is
too slow for 4096 x 14336 units): every unit of the sampled parameters -- the
orthogonalized update O (read back through update_out) per unit and per
256 x 256 block, the stored weight change and the momentum -- and the AdamW
fallback on every element, streamed through the reference in row chunks.
The Llama-3-8B-shaped set samples one parameter of each of its seven shapes;
the MoE set samples units at the first, last and quartile positions of every
bucket, which covers the first and last unit of each bucket and at least one
unit of every chunk the planner cuts a bucket into.  The wide/tall set runs
with both Newton-Schulz methods on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import BLOCK_TOL_BF16, StepRunner, block_rel_max, dev, f64, hp_from, rel, stored
from workloads import configs, gen

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
ADAM_ROWS = 4096  # rows of an AdamW parameter per reference chunk


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
    """One Muon parameter (all its units) against the reference run on it
    alone: O per unit and per block, the weight change and the momentum."""
    row = wl.table[p]
    ref = oracle.muon_step([row], [W0], [G], [np.zeros_like(W0)], [None], [None], _oracle_hp(wl.hp),
                           method=method, want_updates=True)
    worst = worst_blk = 0.0
    for ui, u in enumerate(ref["units"]):
        r0, r1 = u.row0, u.row0 + u.rows
        e = rel(O[r0:r1], ref["O"][ui])
        eb = block_rel_max(O[r0:r1], ref["O"][ui])
        worst, worst_blk = max(worst, e), max(worst_blk, eb)
        assert e <= TOL_BF16, (wl.names[p], ui, e)
        assert eb <= BLOCK_TOL_BF16, (wl.names[p], ui, eb)
    dw_ref = stored(ref["W"][0], torch.bfloat16) - W0
    assert rel(W1 - W0, dw_ref) <= TOL_BF16, (wl.names[p], rel(W1 - W0, dw_ref))
    assert rel(M1, ref["M"][0]) <= 1e-6
    return worst, worst_blk


def _ulp_bf16(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


def _check_adamw_param(name, hp, W0d, Gd, W1d, EAd, ESd):
    """Every element of one AdamW parameter, ADAM_ROWS rows at a time: the
    moments to 1e-6 relative element by element, the stored weight within one
    bf16 rounding (plus the fp32 evaluation error where terms cancel) of the
    reference's, and each chunk's weight change to 2e-2."""
    rows = W0d.shape[0]
    step_u = hp.adam_lr * np.sqrt(1 - hp.adam_beta2) / (1 - hp.adam_beta1)
    for r0 in range(0, rows, ADAM_ROWS):
        sl = slice(r0, min(rows, r0 + ADAM_ROWS))
        w0, g = f64(W0d[sl]), f64(Gd[sl])
        z = np.zeros_like(w0)
        W, m, v = oracle.adamw_update(w0, g, z, z, 1, hp.adam_lr, hp.adam_beta1, hp.adam_beta2,
                                      hp.adam_eps, hp.adam_weight_decay)
        m1, v1, w1 = f64(EAd[sl]), f64(ESd[sl]), f64(W1d[sl])
        assert np.all(np.abs(m1 - m) <= 1e-6 * np.abs(m)), (name, r0)
        assert np.all(np.abs(v1 - v) <= 1e-6 * np.abs(v)), (name, r0)
        Ws = stored(W, torch.bfloat16)
        err = np.abs(w1 - Ws)
        assert np.all(err <= 1.001 * _ulp_bf16(W) + 4 * 2.0 ** -24 * (np.abs(w0) + step_u)), (name, r0)
        assert rel(w1 - w0, Ws - w0) <= TOL_BF16, (name, r0)


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
    A0 = {p: P[p].clone() for p in adam}  # on the GPU until checked
    print(f"full-size {wl.name}: muon_step over {len(wl.table)} parameters", flush=True)
    StepRunner(wl.table, method=method, device=d).step(P, G, M, EA, ES, hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    worst = worst_blk = 0.0
    for p in sel:
        print(f"  reference on {wl.names[p]} {wl.table[p][2]}x{wl.table[p][3]}", flush=True)
        e, eb = _check_muon_param(wl, p, W0[p], Gh[p], f64(P[p]), f64(M[p]), f64(outs[p]))
        worst, worst_blk = max(worst, e), max(worst_blk, eb)
    hp = _oracle_hp(wl.hp)
    for p in adam:
        if wl.table[p][2] > 1:
            print(f"  AdamW reference on every element of {wl.names[p]}", flush=True)
        _check_adamw_param(wl.names[p], hp, A0[p], G[p], P[p], EA[p], ES[p])
    print(f"full-size {wl.name}: worst unit O rel err {worst:.3e}, worst block {worst_blk:.3e}", flush=True)
    del P, G, M, EA, ES, outs, A0
    torch.cuda.empty_cache()


def test_llama3_8b_full_size():
    """One parameter of each of the seven shapes (q, k, v, o, gate, up, down;
    layers spread over the set) plus layer 31's down, and every AdamW
    element (embedding, lm_head, 65 norm vectors)."""
    wl = configs.llama3_8b()
    _run_and_check(wl, 4, ["l0.q", "l7.k", "l31.v", "l19.o", "l12.gate", "l5.up", "l0.down", "l31.down"])


def _moe_sample(wl):
    """Parameters holding the units at positions 0, 1/4, 1/2, 3/4 and the end
    of every bucket of the plan (bucket order), so every bucket's first and
    last unit and every chunk of at least a quarter of a bucket is sampled."""
    plan = mo.muon_plan_create(wl.table, 0)
    units = mo.muon_plan_units(plan)
    names = []
    for (_m, _n, _t, _pd, _cd, _me, first, count) in mo.muon_plan_buckets(plan):
        for q in (0, 1, 2, 3, 4):
            i = first + (q * (count - 1)) // 4
            nm = wl.names[units[i][0]]
            if nm not in names:
                names.append(nm)
    return names


def test_moe_full_size():
    wl = configs.moe_grouped()
    sample = _moe_sample(wl)
    print(f"MoE sample: {sample}", flush=True)
    _run_and_check(wl, 5, sample)


def test_wide_gram_both_methods_full_size():
    """32 wide 4096x14336 and 32 tall 14336x4096 units, once with the Gram
    variant and once with the standard method on the same inputs: sampled
    units against the reference, and the two methods' O on every unit."""
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
            print(f"  reference on {wl.names[p]} ({name})", flush=True)
            _check_muon_param(wl, p, W0[p], Gh[p], f64(Pm[p]), f64(Mm[p]), f64(outs[p]))
        O[name] = outs
        del Pm, Mm
    agree = max(float((a - b).norm() / b.norm()) for a, b in zip(O["gram"], O["standard"]))
    print(f"full-size wide set: max over units of |O_gram - O_std| / |O_std| = {agree:.3e}", flush=True)
    assert agree <= 2 * TOL_BF16
    del P, G, M, O
    torch.cuda.empty_cache()
