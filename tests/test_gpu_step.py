"""GPU parity of muon_step against the fp64 oracle on the small workloads:
the single 256x512 fp32 matrix over three steps (fp32 path, 1e-4) and the
GPT-2-small-shaped set (bf16 path, 2e-2; QKV split blocks, tall MLP-up,
AdamW embedding and vectors).  Momentum and AdamW moments are compared at
1e-6 relative; the orthogonalized update O of every checked unit is read
back through update_out."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import StepRunner, dev, f64, hp_from, rel, stored
from workloads import configs, gen

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu


def _state(wl, device):
    params, moms, eas, ess = gen.make_state(wl, "cpu")
    to = lambda xs: [None if x is None else x.to(device) for x in xs]
    return to(params), to(moms), to(eas), to(ess)


def _oracle_hp(d, adam_step=1):
    return oracle.OracleHparams(lr=d["lr"], momentum=d["momentum"], weight_decay=d["weight_decay"],
                                nesterov=d["nesterov"], ns_steps=d["ns_steps"], adam_lr=d["adam_lr"],
                                adam_beta1=d["adam_beta1"], adam_beta2=d["adam_beta2"],
                                adam_eps=d["adam_eps"], adam_weight_decay=d["adam_weight_decay"],
                                adam_step=adam_step)


def test_single_fp32_three_steps():
    print("muon_step single_256x512_fp32", flush=True)
    d = dev()
    wl = configs.single_256x512()
    P, M, EA, ES = _state(wl, d)
    run = StepRunner(wl.table, device=d)
    W_ref = [f64(P[0])]
    M_ref = [f64(M[0])]
    for step in range(wl.steps):
        G = gen.make_grads(wl, step, "cpu")
        Gd = [g.to(d) for g in G]
        O = torch.zeros(256, 512, dtype=torch.float32, device=d)
        W_old = f64(P[0])
        run.step(P, Gd, M, EA, ES, hp_from(wl.hp), update_outs=[O])
        torch.cuda.synchronize()
        out = oracle.muon_step(wl.table, W_ref, [f64(G[0])], M_ref, [None], [None], _oracle_hp(wl.hp),
                               want_updates=True)
        W_ref, M_ref = out["W"], out["M"]
        assert rel(f64(O), out["O"][0]) <= 1e-4
        assert rel(f64(M[0]), M_ref[0]) <= 1e-6
        assert rel(f64(P[0]) - W_old, W_ref[0] - W_old) <= 1e-4
        assert rel(f64(P[0]), W_ref[0]) <= 1e-6


def test_gpt2_small_bf16_sampled():
    print("muon_step gpt2_small_bf16", flush=True)
    d = dev()
    wl = configs.gpt2_small()
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    Gd = [g.to(d) for g in G]
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) if r[0] == 0 else None
            for r in wl.table]
    W0 = [f64(p) for p in P]
    run = StepRunner(wl.table, device=d)
    run.step(P, Gd, M, EA, ES, hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    # oracle on layers 0 and 11 (qkv blocks, attn-out, tall mlp-up, mlp-down)
    units = oracle.plan_units(wl.table)
    sel = [i for i, u in enumerate(units) if u.param < 4 or 44 <= u.param < 48]
    Wg = [f64(p) if r[0] == 0 else None for p, r in zip(P, wl.table)]
    zeros_muon = [np.zeros((r[2], r[3])) if r[0] == 0 else None for r in wl.table]
    ref = oracle.muon_step(wl.table, W0, [f64(g) for g in G], zeros_muon,
                           [np.zeros((r[2], r[3])) if r[0] == 1 else None for r in wl.table],
                           [np.zeros((r[2], r[3])) if r[0] == 1 else None for r in wl.table],
                           _oracle_hp(wl.hp), units_subset=sel, want_updates=True)
    worst = 0.0
    for ui in sel:
        u = units[ui]
        r0, r1 = u.row0, u.row0 + u.rows
        o = f64(outs[u.param])[r0:r1]
        e = rel(o, ref["O"][ui])
        worst = max(worst, e)
        assert e <= 2e-2, (ui, e)
        dw = Wg[u.param][r0:r1] - W0[u.param][r0:r1]
        dw_ref = stored(ref["W"][u.param][r0:r1], torch.bfloat16) - W0[u.param][r0:r1]
        assert rel(dw, dw_ref) <= 2e-2, (ui, rel(dw, dw_ref))
        assert rel(f64(M[u.param])[r0:r1], ref["M"][u.param][r0:r1]) <= 1e-6
    print("worst unit O rel err", worst)
    # AdamW: every element of the embedding and vectors
    for p, r in enumerate(wl.table):
        if r[0] != 1:
            continue
        assert rel(f64(EA[p]), ref["exp_avg"][p]) <= 1e-6
        assert rel(f64(ES[p]), ref["exp_avg_sq"][p]) <= 1e-6
        assert rel(f64(P[p]) - W0[p], stored(ref["W"][p], torch.bfloat16) - W0[p]) <= 2e-2


def test_grouped_equals_single_and_resume():
    """A unit computed inside a grouped launch is bit-identical to the same
    unit planned alone; two steps equal one step, copy of state, one step."""
    d = dev()
    table = [(0, 1, 384, 640, 0, 0)] * 5
    wl = configs.Workload("five", table, [f"w{i}" for i in range(5)], rank=8, hp=configs._hp())
    P, M, EA, ES = _state(wl, d)
    G = [g.to(d) for g in gen.make_grads(wl, 0, "cpu")]
    outs = [torch.zeros(384, 640, dtype=torch.float32, device=d) for _ in range(5)]
    StepRunner(table, device=d).step([p.clone() for p in P], G, [m.clone() for m in M], EA, ES,
                                     hp_from(wl.hp), update_outs=outs)
    one = StepRunner(table[:1], device=d)
    for i in range(5):
        o = torch.zeros(384, 640, dtype=torch.float32, device=d)
        one.step([P[i].clone()], [G[i]], [M[i].clone()], [None], [None], hp_from(wl.hp), update_outs=[o])
        torch.cuda.synchronize()
        assert torch.equal(o, outs[i])
    # resume: state copied between steps gives the identical trajectory
    run = StepRunner(table, device=d)
    Pa, Ma = [p.clone() for p in P], [m.clone() for m in M]
    Pb, Mb = [p.clone() for p in P], [m.clone() for m in M]
    G2 = [g.to(d) for g in gen.make_grads(wl, 1, "cpu")]
    run.step(Pa, G, Ma, EA, ES, hp_from(wl.hp))
    run.step(Pa, G2, Ma, EA, ES, hp_from(wl.hp))
    run.step(Pb, G, Mb, EA, ES, hp_from(wl.hp))
    Pc = [p.cpu().clone().to(d) for p in Pb]
    Mc = [m.cpu().clone().to(d) for m in Mb]
    StepRunner(table, device=d).step(Pc, G2, Mc, EA, ES, hp_from(wl.hp))
    torch.cuda.synchronize()
    for a, b in zip(Pa, Pc):
        assert torch.equal(a, b)
    for a, b in zip(Ma, Mc):
        assert torch.equal(a, b)


def test_non_nesterov_and_zero_gradient_unit():
    d = dev()
    table = [(0, 0, 96, 160, 0, 0), (0, 0, 64, 64, 0, 0)]
    wl = configs.Workload("nn", table, ["a", "z"], rank=4, hp=configs._hp(nesterov=False))
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    G[1] = torch.zeros_like(G[1])
    W0 = [f64(p) for p in P]
    StepRunner(table, device=d).step(P, [g.to(d) for g in G], M, EA, ES, hp_from(wl.hp))
    torch.cuda.synchronize()
    ref = oracle.muon_step(table, W0, [f64(g) for g in G], [np.zeros((96, 160)), np.zeros((64, 64))],
                           [None, None], [None, None], _oracle_hp(wl.hp))
    assert rel(f64(P[0]) - W0[0], ref["W"][0] - W0[0]) <= 1e-4
    # zero gradient: O = 0, the weight only decays
    assert rel(f64(P[1]), W0[1] * (1 - wl.hp["lr"] * wl.hp["weight_decay"])) <= 1e-6


@pytest.mark.parametrize("pdt,ns_dtype", [(0, 1), (1, 0)])
def test_mixed_precision_parameters(pdt, ns_dtype):
    """fp32 parameters with bf16 Newton-Schulz (2e-2) and bf16 parameters with
    fp32 Newton-Schulz (1e-4 on O), a wide and a tall unit each."""
    print(f"muon_step mixed pdt={pdt} ns_dtype={ns_dtype}", flush=True)
    d = dev()
    table = [(0, pdt, 512, 1536, 0, 0), (0, pdt, 1536, 512, 0, 0)]
    wl = configs.Workload("mixed", table, ["wide", "tall"], rank=8, hp=configs._hp())
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    W0 = [f64(p) for p in P]
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) for r in table]
    StepRunner(table, ns_dtype=ns_dtype, device=d).step(P, [g.to(d) for g in G], M, EA, ES,
                                                       hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    ref = oracle.muon_step(table, W0, [f64(g) for g in G], [np.zeros((r[2], r[3])) for r in table],
                           [None, None], [None, None], _oracle_hp(wl.hp), want_updates=True)
    tol_o = 2e-2 if ns_dtype == 1 else 1e-4
    for i in range(2):
        assert rel(f64(outs[i]), ref["O"][i]) <= tol_o, (i, rel(f64(outs[i]), ref["O"][i]))
        w_ref = ref["W"][i] if pdt == 0 else stored(ref["W"][i], torch.bfloat16)
        tol_w = tol_o if pdt == 0 else 2e-2
        assert rel(f64(P[i]) - W0[i], w_ref - W0[i]) <= tol_w
        assert rel(f64(M[i]), ref["M"][i]) <= 1e-6


@pytest.mark.parametrize("mode,gamma,sched", [("spectral", 1.0, "quintic"), ("unit_rms", 0.18, "hybrid"),
                                               ("moonlight", 2.0, "hybrid")])
def test_scale_modes_and_hybrid_schedule(mode, gamma, sched):
    """Update-scale modes with an extra factor, and the ten-step hybrid
    schedule (eight quintic steps, two refining ones), on a wide and a tall
    bf16 unit."""
    print(f"muon_step scale_mode={mode} gamma={gamma} schedule={sched}", flush=True)
    d = dev()
    table = [(0, 1, 512, 1536, 0, 0), (0, 1, 1536, 512, 0, 0)]
    hpd = configs._hp(ns_steps=10 if sched == "hybrid" else 5)
    wl = configs.Workload("modes", table, ["wide", "tall"], rank=8, hp=hpd)
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    W0 = [f64(p) for p in P]
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) for r in table]
    kind = mo.MUON_COEFF_HYBRID if sched == "hybrid" else mo.MUON_COEFF_QUINTIC
    coeffs = mo.muon_ns_coefficients(kind, hpd["ns_steps"])
    code = {"moonlight": mo.MUON_SCALE_MOONLIGHT, "spectral": mo.MUON_SCALE_SPECTRAL,
            "unit_rms": mo.MUON_SCALE_UNIT_RMS}[mode]
    hp = mo.make_hparams(lr=hpd["lr"], momentum=hpd["momentum"], weight_decay=hpd["weight_decay"],
                         nesterov=hpd["nesterov"], ns_steps=hpd["ns_steps"], coeffs=coeffs,
                         scale_mode=code, extra_scale=gamma)
    StepRunner(table, device=d).step(P, [g.to(d) for g in G], M, EA, ES, hp, update_outs=outs)
    torch.cuda.synchronize()
    ohp = _oracle_hp(hpd)
    ohp.coeffs = oracle.hybrid_schedule(10) if sched == "hybrid" else None
    ohp.scale_mode, ohp.extra_scale = mode, gamma
    ref = oracle.muon_step(table, W0, [f64(g) for g in G], [np.zeros((r[2], r[3])) for r in table],
                           [None, None], [None, None], ohp, want_updates=True)
    for i, r in enumerate(table):
        assert rel(f64(outs[i]), ref["O"][i]) <= 2e-2, (i, rel(f64(outs[i]), ref["O"][i]))
        # the stored weight is W (1 - lr wd) - lr scale O with the GPU's own O
        # and the oracle's scale, rounded to bf16: equal up to one bf16 ulp
        # (the fp32 rounding decision).  A comparison of dW with the oracle's
        # is not meaningful here: at spectral scale the step is a few ulps of W.
        scale = oracle.muon_scale(r[2], r[3], 0, 0.2, mode, gamma)
        w_exp = W0[i] * (1.0 - hpd["lr"] * hpd["weight_decay"]) - hpd["lr"] * scale * f64(outs[i])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(w_exp), 1e-30))) - 7)
        # plus the fp32 evaluation error, which matters where the two terms cancel
        f32err = 4 * 2.0 ** -24 * (np.abs(W0[i]) + hpd["lr"] * scale * np.abs(f64(outs[i])))
        err = np.abs(f64(P[i]) - stored(w_exp, torch.bfloat16))
        assert np.all(err <= 1.01 * ulp + f32err), float(np.max(err - 1.01 * ulp - f32err))


def test_auto_method_mixed_plan():
    """One plan with ns_method auto: the wide and tall units resolve to the
    Gram variant (n/m = 2, m = 512), the square one to the standard method;
    every unit against the oracle."""
    print("muon_step ns_method=auto", flush=True)
    d = dev()
    table = [(0, 1, 512, 1024, 0, 0), (0, 1, 512, 512, 0, 0), (0, 1, 1024, 512, 0, 0)]
    wl = configs.Workload("auto", table, ["wide", "square", "tall"], rank=8, hp=configs._hp())
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    W0 = [f64(p) for p in P]
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) for r in table]
    run = StepRunner(table, method=mo.MUON_NS_AUTO, device=d)
    assert [b[5] for b in mo.muon_plan_buckets(run.plan)] == [1, 0, 1]
    run.step(P, [g.to(d) for g in G], M, EA, ES, hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    ref = oracle.muon_step(table, W0, [f64(g) for g in G], [np.zeros((r[2], r[3])) for r in table],
                           [None] * 3, [None] * 3, _oracle_hp(wl.hp), want_updates=True)
    for i in range(3):
        assert rel(f64(outs[i]), ref["O"][i]) <= 2e-2, (i, rel(f64(outs[i]), ref["O"][i]))
        dw_ref = stored(ref["W"][i], torch.bfloat16) - W0[i]
        assert rel(f64(P[i]) - W0[i], dw_ref) <= 2e-2


def test_empty_parameters_in_the_table():
    """Empty Muon and AdamW parameters (null data pointers) are skipped: the
    other parameters come out bit-identical to a table without them."""
    print("muon_step with empty parameters", flush=True)
    d = dev()
    full = [(0, 1, 0, 96, 0, 0), (0, 1, 256, 384, 0, 0), (1, 1, 1, 0, 0, 0), (1, 1, 1, 256, 0, 0)]
    kept = [full[1], full[3]]
    wl = configs.Workload("e", kept, ["w", "b"], rank=4, hp=configs._hp())
    P, M, EA, ES = _state(wl, d)
    G = [g.to(d) for g in gen.make_grads(wl, 0, "cpu")]
    Pa, Ma = [p.clone() for p in P], [m.clone() if m is not None else None for m in M]
    EAa, ESa = [x.clone() if x is not None else None for x in EA], [x.clone() if x is not None else None for x in ES]
    StepRunner(kept, device=d).step(P, G, M, EA, ES, hp_from(wl.hp))
    e16 = lambda r, c: torch.empty(r, c, dtype=torch.bfloat16, device=d)
    e32 = lambda r, c: torch.empty(r, c, dtype=torch.float32, device=d)
    StepRunner(full, device=d).step([e16(0, 96), Pa[0], e16(1, 0), Pa[1]],
                                    [e16(0, 96), G[0], e16(1, 0), G[1]],
                                    [e32(0, 96), Ma[0], None, None],
                                    [None, None, e32(1, 0), EAa[1]], [None, None, e32(1, 0), ESa[1]],
                                    hp_from(wl.hp))
    torch.cuda.synchronize()
    assert torch.equal(Pa[0], P[0]) and torch.equal(Pa[1], P[1])
    assert torch.equal(Ma[0], M[0]) and torch.equal(EAa[1], EA[1]) and torch.equal(ESa[1], ES[1])
