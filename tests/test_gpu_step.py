"""GPU parity of muon_step against the fp64 oracles on the small workloads.

The single 256x512 fp32 matrix over three steps (fp32 path, 1e-4) and every
one of the 72 units of the GPT-2-small-shaped set (bf16 path, 2e-2 per unit
and 5e-2 per 256 x 256 block; QKV split blocks, tall MLP-up, AdamW embedding
and vectors, every AdamW element) are checked against the plain C++
reference (oracle/muon_ref.cpp through oracle/cref.py).  Momentum and AdamW
moments are compared at 1e-6 relative; the orthogonalized update O of every
checked unit is read back through update_out.  Further cases (mixed
precision, scale modes, schedules, ragged unaligned buffers, a NaN-filled
workspace) use the numpy reference."""
import numpy as np
import pytest
import torch

import oracle
from oracle import cref
from tests.gpu_util import (BLOCK_TOL_BF16, StepRunner, block_rel_max, dev, f64, hp_from, rel,
                            stored)
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
    """The 256 x 512 fp32 matrix, three steps with a fresh gradient each,
    against the C++ reference carried along the same three steps."""
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
        out = cref.muon_step(wl.table, W_ref, [f64(G[0])], M_ref, [None], [None], _oracle_hp(wl.hp),
                             want_updates=True)
        W_ref, M_ref = out["W"], out["M"]
        assert rel(f64(O), out["O"][0]) <= 1e-4
        assert rel(f64(M[0]), M_ref[0]) <= 1e-6
        assert rel(f64(P[0]) - W_old, W_ref[0] - W_old) <= 1e-4
        assert rel(f64(P[0]), W_ref[0]) <= 1e-6


@pytest.fixture(scope="module")
def gpt2_run():
    """One muon_step over the whole GPT-2-small-shaped table on the GPU; the
    inputs and every output come back to the host (as torch CPU tensors)."""
    print("muon_step gpt2_small_bf16 (whole table)", flush=True)
    d = dev()
    wl = configs.gpt2_small()
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) if r[0] == 0 else None
            for r in wl.table]
    W0 = [p.cpu() for p in P]
    StepRunner(wl.table, device=d).step(P, [g.to(d) for g in G], M, EA, ES, hp_from(wl.hp),
                                        update_outs=outs)
    torch.cuda.synchronize()
    host = lambda xs: [None if x is None else x.cpu() for x in xs]
    return {"wl": wl, "W0": W0, "G": G, "W1": host(P), "M1": host(M), "O": host(outs),
            "EA": host(EA), "ES": host(ES)}


GPT2_GROUPS = 6


@pytest.mark.parametrize("group", range(GPT2_GROUPS))
def test_gpt2_small_every_unit(gpt2_run, group):
    """Units group, group + 6, ... of the 72 (every layer's Q, K, V blocks,
    attn-out, tall MLP-up and MLP-down across the six groups) against the
    C++ reference: O per unit and per block, the stored weight change and
    the momentum."""
    r = gpt2_run
    wl = r["wl"]
    units = cref.units_in_table_order(wl.table)
    assert len(units) == 72
    sel = [i for i in range(len(units)) if i % GPT2_GROUPS == group]
    touched = {units[i].param for i in sel}
    pick = lambda xs: [f64(x) if p in touched and x is not None else None for p, x in enumerate(xs)]
    zeros = [np.zeros((t[2], t[3])) if p in touched else None for p, t in enumerate(wl.table)]
    print(f"C++ reference on {len(sel)} units of group {group}", flush=True)
    ref = cref.muon_step(wl.table, pick(r["W0"]), pick(r["G"]), zeros, [None] * len(wl.table),
                         [None] * len(wl.table), _oracle_hp(wl.hp), units_subset=sel, want_updates=True,
                         adamw_params=False)
    worst = 0.0
    for ui in sel:
        u = units[ui]
        r0, r1 = u.row0, u.row0 + u.rows
        o = f64(r["O"][u.param][r0:r1])
        e = rel(o, ref["O"][ui])
        worst = max(worst, e)
        assert e <= 2e-2, (ui, wl.names[u.param], e)
        eb = block_rel_max(o, ref["O"][ui])
        assert eb <= BLOCK_TOL_BF16, (ui, wl.names[u.param], eb)
        w0 = f64(r["W0"][u.param][r0:r1])
        dw = f64(r["W1"][u.param][r0:r1]) - w0
        dw_ref = stored(ref["W"][u.param][r0:r1], torch.bfloat16) - w0
        assert rel(dw, dw_ref) <= 2e-2, (ui, rel(dw, dw_ref))
        assert rel(f64(r["M1"][u.param][r0:r1]), ref["M"][u.param][r0:r1]) <= 1e-6
    print(f"group {group}: worst unit O rel err {worst:.3e}", flush=True)


def _ulp_bf16(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


def test_gpt2_small_adamw_every_element(gpt2_run):
    """Every element of the 50257 x 768 embedding and the 74 vectors against
    the C++ reference's AdamW: moments to 1e-6 relative element by element,
    the stored weight within one bf16 rounding of the reference's new weight
    (the fp32 evaluation can land on the other side of a rounding midpoint)
    and its change to 2e-2 overall."""
    r = gpt2_run
    wl = r["wl"]
    hp = _oracle_hp(wl.hp)
    for p, row in enumerate(wl.table):
        if row[0] != 1:
            continue
        w0, g = f64(r["W0"][p]), f64(r["G"][p])
        z = np.zeros_like(w0)
        W, m, v = cref.adamw(w0, g, z, z, 1, hp.adam_lr, hp.adam_beta1, hp.adam_beta2, hp.adam_eps,
                             hp.adam_weight_decay)
        m1, v1, w1 = f64(r["EA"][p]), f64(r["ES"][p]), f64(r["W1"][p])
        assert np.all(np.abs(m1 - m) <= 1e-6 * np.abs(m)), wl.names[p]
        assert np.all(np.abs(v1 - v) <= 1e-6 * np.abs(v)), wl.names[p]
        # plus the fp32 evaluation error of W (1 - lr wd) - step u, which
        # matters where the two terms cancel (|step u| <= lr sqrt(1-b2)/(1-b1))
        step_u = hp.adam_lr * np.sqrt(1 - hp.adam_beta2) / (1 - hp.adam_beta1)
        f32err = 4 * 2.0 ** -24 * (np.abs(w0) + step_u)
        err = np.abs(w1 - stored(W, torch.bfloat16))
        assert np.all(err <= 1.001 * _ulp_bf16(W) + f32err), (wl.names[p], float(np.max(err - _ulp_bf16(W))))
        assert rel(w1 - w0, stored(W, torch.bfloat16) - w0) <= 2e-2


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
    Gram variant (n/m = 3, m = 512), the square one to the standard method;
    every unit against the oracle."""
    print("muon_step ns_method=auto", flush=True)
    d = dev()
    table = [(0, 1, 512, 1536, 0, 0), (0, 1, 512, 512, 0, 0), (0, 1, 1536, 512, 0, 0)]
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


def _offset_tensor(rows, cols, dtype, device, fill=None):
    """A contiguous rows x cols tensor whose data starts one element into its
    storage, so that its rows are not 16-byte aligned."""
    buf = torch.zeros(rows * cols + 1, dtype=dtype, device=device)
    t = buf[1:].view(rows, cols)
    if fill is not None:
        t.copy_(fill)
    return t


@pytest.mark.parametrize("pdt", [0, 1])
def test_ragged_unaligned_buffers(pdt):
    """Unaligned parameter, gradient, momentum and update_out buffers (storage
    offset of one element) with ragged shapes, a wide 300 x 701 and a tall
    701 x 300 unit, and an AdamW parameter of 1001 elements: the element-wise
    load/store paths of the momentum, fused-update and AdamW kernels; the
    wide unit carries a scale_dim override.  W, M, O, m and v against the
    numpy reference."""
    print(f"muon_step ragged unaligned pdt={pdt}", flush=True)
    d = dev()
    # the wide unit also overrides the scale dimension (scale 0.2 sqrt(1000))
    table = [(0, pdt, 300, 701, 0, 1000), (0, pdt, 701, 300, 0, 0), (1, pdt, 1, 1001, 0, 0)]
    wl = configs.Workload("ragged", table, ["wide", "tall", "vec"], rank=8, hp=configs._hp())
    P0, M0, EA0, ES0 = gen.make_state(wl, "cpu")
    G0 = gen.make_grads(wl, 0, "cpu")
    tdt = gen.torch_dtype(pdt)
    P = [_offset_tensor(r[2], r[3], tdt, d, p) for r, p in zip(table, P0)]
    G = [_offset_tensor(r[2], r[3], tdt, d, g) for r, g in zip(table, G0)]
    M = [_offset_tensor(r[2], r[3], torch.float32, d) if r[0] == 0 else None for r in table]
    EA = [_offset_tensor(r[2], r[3], torch.float32, d) if r[0] == 1 else None for r in table]
    ES = [_offset_tensor(r[2], r[3], torch.float32, d) if r[0] == 1 else None for r in table]
    O = [_offset_tensor(r[2], r[3], torch.float32, d) if r[0] == 0 else None for r in table]
    assert all(t.data_ptr() % 16 != 0 for t in P + G + [M[0], M[1], O[0], O[1], EA[2], ES[2]])
    StepRunner(table, device=d).step(P, G, M, EA, ES, hp_from(wl.hp), update_outs=O)
    torch.cuda.synchronize()
    W0 = [f64(p) for p in P0]
    ref = oracle.muon_step(table, W0, [f64(g) for g in G0],
                           [np.zeros((r[2], r[3])) if r[0] == 0 else None for r in table],
                           [None, None, np.zeros((1, 1001))], [None, None, np.zeros((1, 1001))],
                           _oracle_hp(wl.hp), want_updates=True)
    tol = 1e-4 if pdt == 0 else 2e-2
    for i in range(2):
        assert rel(f64(O[i]), ref["O"][i]) <= tol, (i, rel(f64(O[i]), ref["O"][i]))
        w_ref = ref["W"][i] if pdt == 0 else stored(ref["W"][i], torch.bfloat16)
        assert rel(f64(P[i]) - W0[i], w_ref - W0[i]) <= tol
        assert rel(f64(M[i]), ref["M"][i]) <= 1e-6
    assert rel(f64(EA[2]), ref["exp_avg"][2]) <= 1e-6
    assert rel(f64(ES[2]), ref["exp_avg_sq"][2]) <= 1e-6
    w_ref = ref["W"][2] if pdt == 0 else stored(ref["W"][2], torch.bfloat16)
    assert rel(f64(P[2]) - W0[2], w_ref - W0[2]) <= tol


def _run_with_workspace(table, wl, fill_byte, device, method=0):
    """One step from fixed inputs with the workspace pre-filled with a byte
    pattern; returns every output on the host."""
    P, M, EA, ES = _state(wl, device)
    G = [g.to(device) for g in gen.make_grads(wl, 0, "cpu")]
    O = [torch.zeros(r[2], r[3], dtype=torch.float32, device=device) if r[0] == 0 else None
         for r in table]
    run = StepRunner(table, method=method, device=device)
    run.ws.fill_(fill_byte)
    run.step(P, G, M, EA, ES, hp_from(wl.hp), update_outs=O)
    torch.cuda.synchronize()
    host = lambda xs: [None if x is None else x.cpu() for x in xs]
    return host(P) + host(M) + host(EA) + host(ES) + host(O)


@pytest.mark.parametrize("which,method", [("gpt2_small", 0), ("ragged", 0), ("ragged", 1), ("ragged", 3)])
def test_nan_filled_workspace(which, method):
    """Every GEMM reads whole 16-byte pieces and relies on the zero padding of
    the working copies being written by the kernels themselves.  A workspace
    filled with 0xFF bytes (NaN in bf16 and fp32) before the step must give
    bit-identical results to a zero-filled one: the standard method, the Gram
    chain (fp16, fp32 and the standard method for fp32 units) and the
    restarted chain, whose restart iterate X_r is one more working copy."""
    print(f"muon_step with a NaN-filled workspace: {which}, method {method}", flush=True)
    d = dev()
    if which == "gpt2_small":
        wl = configs.gpt2_small()
    else:
        table = [(0, 1, 300, 701, 0, 0), (0, 1, 701, 300, 0, 0), (0, 1, 200, 130, 0, 0),
                 (0, 0, 77, 190, 0, 0), (1, 1, 1, 1001, 0, 0), (0, 1, 514, 1550, 0, 0)]
        wl = configs.Workload("ragged", table, [f"p{i}" for i in range(6)], rank=8, hp=configs._hp())
    a = _run_with_workspace(wl.table, wl, 0, d, method)
    b = _run_with_workspace(wl.table, wl, 0xFF, d, method)
    for x, y in zip(a, b):
        if x is not None:
            assert torch.equal(x, y)
            assert torch.isfinite(x.float()).all()


def test_restarted_gram_step():
    """One muon_step with the restarted Gram chain over wide, tall, square and
    small units (the fp16 chain with its restart for m >= 256, the fp32
    Gram chain for 96 x 300) and an fp32 unit (resolved as a Gram request:
    the standard method outside m >= 512, n >= 3m): O, W and M of every unit
    against the numpy reference."""
    print("muon_step ns_method=gram_restart", flush=True)
    d = dev()
    table = [(0, 1, 512, 1536, 0, 0), (0, 1, 1536, 512, 0, 0), (0, 1, 256, 1024, 0, 0), (0, 1, 640, 640, 0, 0),
             (0, 1, 96, 300, 0, 0), (0, 0, 300, 700, 0, 0)]
    wl = configs.Workload("gram_restart", table, [f"p{i}" for i in range(6)], rank=8, hp=configs._hp())
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    W0 = [f64(p) for p in P]
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) for r in table]
    run = StepRunner(table, method=mo.MUON_NS_GRAM_RESTART, device=d)
    b = mo.muon_plan_buckets(run.plan)
    assert [(x[4], x[5]) for x in b] == [(1, 3), (1, 3), (1, 3), (1, 3), (0, 1), (0, 0)]
    run.step(P, [g.to(d) for g in G], M, EA, ES, hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    ref = oracle.muon_step(table, W0, [f64(g) for g in G], [np.zeros((r[2], r[3])) for r in table],
                           [None] * 6, [None] * 6, _oracle_hp(wl.hp), method="gram_restart", want_updates=True)
    for i, r in enumerate(table):
        tol = 1e-4 if r[1] == 0 else 2e-2
        e = rel(f64(outs[i]), ref["O"][i])
        print(f"  {r[2]}x{r[3]} dtype {r[1]}: O rel err {e:.3e}", flush=True)
        assert e <= tol, (i, e)
        w_ref = ref["W"][i] if r[1] == 0 else stored(ref["W"][i], torch.bfloat16)
        assert rel(f64(P[i]) - W0[i], w_ref - W0[i]) <= tol
        assert rel(f64(M[i]), ref["M"][i]) <= 1e-6


def test_explicit_gram_step_every_precision_path():
    """One muon_step with ns_method gram over units that take each of its
    resolutions: the fp16 chain (512 x 1536 wide and tall), the fp32 chain of
    a bf16 unit outside m >= 512, n >= 3m (256 x 1024, 640 x 640), and an fp32
    parameter outside it, served by the standard method (300 x 700).  Every
    unit against the numpy reference (2e-2 bf16, 1e-4 fp32)."""
    print("muon_step ns_method=gram, every precision path", flush=True)
    d = dev()
    table = [(0, 1, 512, 1536, 0, 0), (0, 1, 1536, 512, 0, 0), (0, 1, 256, 1024, 0, 0), (0, 1, 640, 640, 0, 0),
             (0, 0, 300, 700, 0, 0)]
    wl = configs.Workload("gram", table, [f"p{i}" for i in range(5)], rank=8, hp=configs._hp())
    P, M, EA, ES = _state(wl, d)
    G = gen.make_grads(wl, 0, "cpu")
    W0 = [f64(p) for p in P]
    outs = [torch.zeros(r[2], r[3], dtype=torch.float32, device=d) for r in table]
    run = StepRunner(table, method=mo.MUON_NS_GRAM, device=d)
    b = mo.muon_plan_buckets(run.plan)
    assert [(x[4], x[5]) for x in b] == [(1, 1), (1, 1), (0, 1), (0, 1), (0, 0)]
    run.step(P, [g.to(d) for g in G], M, EA, ES, hp_from(wl.hp), update_outs=outs)
    torch.cuda.synchronize()
    ref = oracle.muon_step(table, W0, [f64(g) for g in G], [np.zeros((r[2], r[3])) for r in table],
                           [None] * 5, [None] * 5, _oracle_hp(wl.hp), want_updates=True)
    for i, r in enumerate(table):
        tol = 1e-4 if r[1] == 0 else 2e-2
        e = rel(f64(outs[i]), ref["O"][i])
        print(f"  {r[2]}x{r[3]} dtype {r[1]}: O rel err {e:.3e}", flush=True)
        assert e <= tol, (i, e)
        w_ref = ref["W"][i] if r[1] == 0 else stored(ref["W"][i], torch.bfloat16)
        assert rel(f64(P[i]) - W0[i], w_ref - W0[i]) <= tol
        assert rel(f64(M[i]), ref["M"][i]) <= 1e-6
