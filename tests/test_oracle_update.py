"""Pins of the oracle's momentum, weight update, AdamW fallback, planner and
whole step against closed forms and hand-reduced 2x3 cases.  The elementwise
pins run on both references (numpy and the plain C++ one)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import cref
from workloads import configs


@pytest.fixture(params=["numpy", "cpp"])
def impl(request):
    return oracle if request.param == "numpy" else cref


def test_momentum_three_steps_closed_form(impl):
    r = np.random.default_rng(0)
    G1, G2, G3 = (r.standard_normal((2, 3)) for _ in range(3))
    mu = 0.95
    M = np.zeros((2, 3))
    for G in (G1, G2):
        M, _ = impl.momentum_update(M, G, mu, True)
    M3, U3 = impl.momentum_update(M, G3, mu, True)
    assert np.allclose(M3, mu * mu * G1 + mu * G2 + G3, atol=1e-15)
    assert np.allclose(U3, G3 + mu * (mu * mu * G1 + mu * G2 + G3), atol=1e-15)
    M3p, U3p = impl.momentum_update(M, G3, mu, False)
    assert np.array_equal(U3p, M3p)


def test_momentum_hand_2x3(impl):
    M = np.array([[1.0, -2.0, 0.5], [0.0, 4.0, -1.0]])
    G = np.array([[0.5, 0.5, 0.5], [-1.0, 0.0, 2.0]])
    Mn, U = impl.momentum_update(M, G, 0.5, True)
    assert np.array_equal(Mn, [[1.0, -0.5, 0.75], [-1.0, 2.0, 1.5]])
    assert np.array_equal(U, [[1.0, 0.25, 0.875], [-1.5, 1.0, 2.75]])


@pytest.mark.parametrize("shape,val", [((256, 512), 4.5255), ((768, 768), 5.5426),
                                       ((14336, 4096), 23.9466), ((1408, 2048), 9.0510)])
def test_scale_values(shape, val, impl):
    assert abs(impl.muon_scale(*shape) - val) < 5e-5
    assert impl.muon_scale(768, 768, scale_dim=2304) == pytest.approx(0.2 * 48.0)


def test_weight_update_hand_2x3(impl):
    W = np.array([[1.0, 2.0, -1.0], [0.0, 0.5, 4.0]])
    O = np.array([[0.5, 0.0, -0.5], [1.0, -1.0, 0.0]])
    lr, wd, s = 0.1, 0.5, 2.0
    # W (1 - 0.05) - 0.2 O
    exp = np.array([[0.85, 1.9, -0.85], [-0.2, 0.675, 3.8]])
    assert np.allclose(impl.weight_update(W, O, lr, wd, s), exp, atol=1e-15)


def test_adamw_step1_closed_form(impl):
    r = np.random.default_rng(4)
    W = r.standard_normal((2, 3))
    g = r.standard_normal((2, 3))
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.95, 1e-8, 0.1
    Wn, m, v = impl.adamw_update(W, g, np.zeros_like(g), np.zeros_like(g), 1, lr, b1, b2, eps, wd)
    k = math.sqrt(1 - b2)
    assert np.allclose(Wn - W, -lr * wd * W - lr * k * g / (eps + k * np.abs(g)), rtol=1e-12, atol=1e-18)
    assert np.allclose(m, (1 - b1) * g) and np.allclose(v, (1 - b2) * g * g)


def test_adamw_step2_hand(impl):
    # scalars: g1 = 2, g2 = -1, beta1 = 0.5, beta2 = 0.75, eps = 0, lr = 1, wd = 0
    W = np.array([[0.0]])
    W1, m, v = impl.adamw_update(W, np.array([[2.0]]), np.zeros((1, 1)), np.zeros((1, 1)),
                                   1, 1.0, 0.5, 0.75, 0.0, 0.0)
    # m1 = 1, v1 = 1, scale = 0.5 / sqrt(0.25) = 1, W1 = -1
    assert W1[0, 0] == pytest.approx(-1.0)
    W2, m, v = impl.adamw_update(W1, np.array([[-1.0]]), m, v, 2, 1.0, 0.5, 0.75, 0.0, 0.0)
    # m2 = 0, v2 = 0.75*1 + 0.25*1 = 1 -> u = 0, W unchanged
    assert m[0, 0] == pytest.approx(0.0) and v[0, 0] == pytest.approx(1.0)
    assert W2[0, 0] == pytest.approx(-1.0)


def test_full_step_hand_2x3(golden_dir, impl):
    with open(os.path.join(golden_dir, "ns_diag_2x3.json")) as f:
        gold = json.load(f)
    G = np.array(gold["G"])
    O = np.array(gold["O"])
    W = np.array([[0.1, -0.2, 0.3], [0.0, 0.5, -0.4]])
    hp = oracle.OracleHparams(lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True)
    table = [(0, 1, 2, 3, 0, 0)]
    out = impl.muon_step(table, [W], [G], [np.zeros((2, 3))], [None], [None], hp,
                         want_updates=True)
    # M1 = G, U = 1.95 G, NS is scale invariant -> O; scale 0.2 sqrt(3)
    assert np.array_equal(out["M"][0], G)
    assert np.allclose(out["O"][0], O, atol=1e-14)
    exp = W * (1 - 0.02 * 0.1) - 0.02 * 0.2 * math.sqrt(3) * O
    assert np.allclose(out["W"][0], exp, atol=1e-15)


def test_split_units_are_independent(impl):
    r = np.random.default_rng(8)
    G = r.standard_normal((6, 4))
    W = r.standard_normal((6, 4))
    hp = oracle.OracleHparams()
    table = [(0, 1, 6, 4, 2, 0)]
    out = impl.muon_step(table, [W], [G], [np.zeros((6, 4))], [None], [None], hp,
                         want_updates=True)
    for b in range(3):
        Ob = impl.orthogonalize((1 + hp.momentum) * G[2 * b:2 * b + 2])
        assert np.allclose(out["O"][b], Ob, atol=1e-14)
        sc = impl.muon_scale(2, 4)
        exp = W[2 * b:2 * b + 2] * (1 - hp.lr * hp.weight_decay) - hp.lr * sc * Ob
        assert np.allclose(out["W"][0][2 * b:2 * b + 2], exp, atol=1e-14)


def test_step_of_both_references_agrees():
    """The whole step over a mixed table (split blocks, a tall unit with a
    scale override, an AdamW vector), numpy reference against C++ one."""
    r = np.random.default_rng(9)
    table = [(0, 0, 12, 5, 4, 0), (0, 0, 9, 4, 0, 13), (1, 0, 1, 7, 0, 0)]
    W = [r.standard_normal((t[2], t[3])) for t in table]
    G = [r.standard_normal((t[2], t[3])) for t in table]
    M = [r.standard_normal((t[2], t[3])) if t[0] == 0 else None for t in table]
    EA = [None, None, r.standard_normal((1, 7))]
    ES = [None, None, r.random((1, 7))]
    hp = oracle.OracleHparams(adam_step=3)
    a = oracle.muon_step(table, W, G, M, EA, ES, hp, want_updates=True)
    b = cref.muon_step(table, W, G, M, EA, ES, hp, want_updates=True)
    for k in ("W", "M", "exp_avg", "exp_avg_sq"):
        for x, y in zip(a[k], b[k]):
            if x is not None:
                assert np.allclose(x, y, rtol=1e-12, atol=1e-14), k
    assert sorted(a["O"]) == sorted(b["O"]) == list(range(4))
    for i in a["O"]:
        assert np.allclose(a["O"][i], b["O"][i], atol=1e-13)


def _bucket_summary(table, method=0, impl=oracle):
    """[(key, count)] per bucket, plus the units in table order (numpy) or
    bucket order (C++), from either reference's planner."""
    if impl is oracle:
        units, keys, members = oracle.plan_buckets(table, method)
        return [(k, len(mem)) for k, mem in zip(keys, members)], units, members
    units, buckets = cref.plan(table, method)
    return [(tuple(b[:6]), b[7]) for b in buckets], units, None


def test_plan_gpt2(impl):
    summ, units, members = _bucket_summary(configs.gpt2_small().table, impl=impl)
    assert len(units) == 12 * 6
    assert summ == [((768, 768, 0, 1, 1, 0), 48), ((768, 3072, 1, 1, 1, 0), 12), ((768, 3072, 0, 1, 1, 0), 12)]
    if members is not None:
        # units keep table order inside a bucket
        for mem in members:
            assert mem == sorted(mem)
        assert [(u.param, u.row0) for u in units[:4]] == [(0, 0), (0, 768), (0, 1536), (1, 0)]
    else:
        assert [tuple(u[:2]) for u in units[:4]] == [(0, 0), (0, 768), (0, 1536), (1, 0)]


def test_plan_llama_and_moe(impl):
    summ, _, _ = _bucket_summary(configs.llama3_8b().table, impl=impl)
    assert summ == [((4096, 4096, 0, 1, 1, 0), 64), ((1024, 4096, 0, 1, 1, 0), 64),
                    ((4096, 14336, 1, 1, 1, 0), 64), ((4096, 14336, 0, 1, 1, 0), 32)]
    summ, units, _ = _bucket_summary(configs.moe_grouped().table, impl=impl)
    assert len(units) == 6656
    assert summ == [((128, 2048, 0, 1, 1, 0), 1664), ((1408, 2048, 0, 1, 1, 0), 3328),
                    ((1408, 2048, 1, 1, 1, 0), 1664)]
    summ, _, _ = _bucket_summary(configs.wide_gram().table, 1, impl=impl)
    assert summ == [((4096, 14336, 0, 1, 1, 1), 32), ((4096, 14336, 1, 1, 1, 1), 32)]


def test_plan_gram_resolution_literal(impl):
    """Method and compute dtype of Gram and auto requests, by hand: Gram's
    fp16 chain only for m >= 512 and n >= 3m; outside, a bf16 request keeps
    Gram in fp32 (dtype 0) and an fp32 request takes the standard method."""
    table = [(0, 1, 512, 1536, 0, 0), (0, 1, 512, 1535, 0, 0), (0, 1, 511, 4096, 0, 0),
             (0, 0, 300, 900, 0, 0), (0, 0, 1024, 4096, 0, 0)]
    summ, _, _ = _bucket_summary(table, 1, impl=impl)
    assert summ == [((512, 1536, 0, 1, 1, 1), 1), ((512, 1535, 0, 1, 0, 1), 1), ((511, 4096, 0, 1, 0, 1), 1),
                    ((300, 900, 0, 0, 0, 0), 1), ((1024, 4096, 0, 0, 0, 1), 1)]
    summ, _, _ = _bucket_summary(table, 2, impl=impl)
    assert [k[4:] for k, _ in summ] == [(1, 1), (1, 0), (1, 0), (0, 0), (0, 1)]
