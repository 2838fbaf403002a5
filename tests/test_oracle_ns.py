"""Pins of the oracle's orthogonalization against what the mathematics fixes:
the SVD closed form of the iteration, hand-reduced and rank-1 cases, the exact
msign limit of convergent coefficient sets, scalar fixed points of g,
symmetries, the Gram rewrite (with and without its restart) and the
singular-value band.  Every test runs on both references: the numpy one and the plain C++ one (oracle/muon_ref.cpp),
which share no code."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import cref

QUINTIC = (3.4445, -4.7750, 2.0315)


@pytest.fixture(params=["numpy", "cpp"])
def impl(request):
    if request.param == "numpy":
        return oracle
    return cref


def rng(seed):
    return np.random.default_rng(seed)


def closed_form(G, steps=5, coeffs=None):
    """U g^N(S/||G||_F) V^T from numpy's SVD (a library routine, independent of
    the oracle's matmul iteration)."""
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = np.linalg.norm(G)
    mapped = np.array([oracle.quintic_scalar(x / s, steps, coeffs) for x in S])
    return (U * mapped) @ Vt


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("shape", [(4, 7), (7, 4), (16, 16), (8, 24), (30, 12), (1, 5), (5, 1)])
def test_matches_svd_closed_form(shape, impl):
    G = rng(shape[0] * 100 + shape[1]).standard_normal(shape)
    O = impl.orthogonalize(G)
    assert O.shape == G.shape
    assert rel(O, closed_form(G)) < 1e-12


@pytest.mark.parametrize("method", ["standard", "gram", "gram_restart"])
def test_lowrank_closed_form(method, impl):
    # a gradient of the workload kind: geometric spectrum 1..1e-3 plus noise
    r = rng(7)
    m, n, k = 24, 40, 6
    s = 10.0 ** (-3.0 * np.arange(k) / (k - 1))
    U = r.standard_normal((m, k))
    U /= np.linalg.norm(U, axis=0)
    V = r.standard_normal((n, k))
    V /= np.linalg.norm(V, axis=0)
    G = (U * s) @ V.T + 1e-3 * r.standard_normal((m, n))
    assert rel(impl.orthogonalize(G, method=method), closed_form(G)) < 1e-10


def test_diag_2x3_golden(golden_dir, impl):
    with open(os.path.join(golden_dir, "ns_diag_2x3.json")) as f:
        gold = json.load(f)
    O = impl.orthogonalize(np.array(gold["G"]))
    assert np.allclose(O, np.array(gold["O"]), rtol=0, atol=1e-14)
    # the transposed (tall) case gives the transposed result
    Ot = impl.orthogonalize(np.array(gold["G"]).T)
    assert np.allclose(Ot, np.array(gold["O"]).T, rtol=0, atol=1e-14)


def test_rank1(golden_dir, impl):
    with open(os.path.join(golden_dir, "ns_diag_2x3.json")) as f:
        g5_1 = json.load(f)["g5_of_1"]
    r = rng(3)
    u = r.standard_normal(9)
    u /= np.linalg.norm(u)
    v = r.standard_normal(13)
    v /= np.linalg.norm(v)
    G = 2.5 * np.outer(u, v)
    assert rel(impl.orthogonalize(G), g5_1 * np.outer(u, v)) < 1e-13


def test_scalar_map_fixed_points():
    # g(x) = x  <=>  (a - 1) + b x^2 + c x^4 = 0: the two positive roots are
    # fixed points of one quintic step, and g(1) = a + b + c.
    a, b, c = QUINTIC
    disc = math.sqrt(b * b - 4 * c * (a - 1))
    for y in ((-b - disc) / (2 * c), (-b + disc) / (2 * c)):
        x = math.sqrt(y)
        assert abs(oracle.quintic_scalar(x, 1) - x) < 1e-12
    assert abs(oracle.quintic_scalar(1.0, 1) - (a + b + c)) < 1e-15
    # derivative at zero is a: the small-x gain after 5 steps is a^5
    eps = 1e-9
    assert abs(oracle.quintic_scalar(eps, 5) / eps - a ** 5) < 1e-6 * a ** 5
    # the Newton step for x^-2 - 1 ([Blog] "Sign of a Matrix") has 1 as fixed point
    assert oracle.quintic_scalar(1.0, 1, (1.5, -0.5, 0.0)) == 1.0


@pytest.mark.parametrize("coeffs,steps", [((1.875, -1.25, 0.375), 40), ((1.5, -0.5, 0.0), 60)])
def test_convergent_coeffs_reach_exact_msign(coeffs, steps, impl):
    # Second-order Taylor of x^-1/2 (the page's -7/8 is read as -5/4, the only
    # value with p(1) = 1) and the Newton iteration converge to U V^T
    # ([Blog] "Orthogonalization of Gradients", theorem: O = U V^T).
    r = rng(11)
    for shape in [(6, 10), (10, 6), (8, 8)]:
        Q1, _ = np.linalg.qr(r.standard_normal((shape[0], shape[0])))
        Q2, _ = np.linalg.qr(r.standard_normal((shape[1], shape[1])))
        k = min(shape)
        S = np.linspace(1.0, 0.3, k)
        G = Q1[:, :k] @ np.diag(S) @ Q2[:, :k].T
        O = impl.orthogonalize(G, steps=steps, coeffs=coeffs)
        U, _, Vt = np.linalg.svd(G, full_matrices=False)
        assert rel(O, U @ Vt) < 1e-10
        # corollary: a semi-orthogonal matrix has ||O||_F^2 = min(m, n)
        assert abs(np.sum(O * O) - min(shape)) < 1e-9


def test_gram_equals_standard(impl):
    r = rng(5)
    for shape in [(12, 40), (40, 12), (16, 16), (3, 50)]:
        G = r.standard_normal(shape)
        a = impl.orthogonalize(G, method="standard")
        b = impl.orthogonalize(G, method="gram")
        assert rel(b, a) < 1e-11


def test_restarted_gram_equals_standard(impl):
    """The restart changes nothing in exact arithmetic: X_r = Q X_0 is the
    standard iterate after r steps and R = X_r X_r^T its Gram matrix.  Any
    step count (the restart sits after ceil(steps / 2) of them), per-step
    coefficients, tall and wide inputs."""
    r = rng(15)
    for shape, steps in [((12, 40), 5), ((40, 12), 5), ((16, 16), 2), ((9, 30), 3), ((20, 33), 10)]:
        G = r.standard_normal(shape)
        coeffs = [(3.4445 - 0.1 * k, -4.7750 + 0.05 * k, 2.0315) for k in range(steps)]
        a = impl.orthogonalize(G, steps=steps, coeffs=coeffs, method="standard")
        b = impl.orthogonalize(G, steps=steps, coeffs=coeffs, method="gram_restart")
        assert rel(b, a) < 1e-11


def test_restart_step():
    assert [oracle.restart_step(s) for s in (0, 1, 2, 3, 5, 10)] == [0, 0, 1, 2, 3, 5]


@pytest.mark.parametrize("shape", [(96, 128), (128, 128)])
def test_restart_cuts_rounded_chain_error(shape):
    """What the restart is for, seen in rounded arithmetic (numpy reference,
    chain in fp32): restarting from the rectangular iterate where the
    library does (after three of the five steps) brings the chain at least
    4x closer to the fp64 standard result than the plain chain.  A restart
    that never happens, or one that loses Q, fails this."""
    m, n = shape
    r = rng(m + n)
    U, _ = np.linalg.qr(r.standard_normal((m, m)))
    V, _ = np.linalg.qr(r.standard_normal((n, m)))
    G = (U * np.geomspace(1.0, 1e-3, m)) @ V.T
    X = G / np.linalg.norm(G)
    ref = oracle.ns_standard(X, [QUINTIC] * 5)
    plain = oracle.ns_gram(X, [QUINTIC] * 5, dtype=np.float32)
    restarted = oracle.ns_gram(X, [QUINTIC] * 5, restart_after=oracle.restart_step(5), dtype=np.float32)
    e_plain, e_rst = rel(plain, ref), rel(restarted, ref)
    assert 1e-5 < e_plain < 1e-3
    assert e_rst * 4 < e_plain
    # and in fp64 both are the standard result
    assert rel(oracle.ns_gram(X, [QUINTIC] * 5, restart_after=2), ref) < 1e-12


def test_per_step_schedule_matches_constant(impl):
    G = rng(2).standard_normal((5, 9))
    a = impl.orthogonalize(G)
    b = impl.orthogonalize(G, coeffs=[QUINTIC] * 5)
    assert np.array_equal(a, b)
    # a non-constant schedule follows the scalar composition
    sched = [QUINTIC] * 3 + [(1.5, -0.5, 0.0)] * 2
    assert rel(impl.orthogonalize(G, coeffs=sched), closed_form(G, 5, sched)) < 1e-12


def test_symmetries(impl):
    r = rng(9)
    G = r.standard_normal((7, 11))
    O = impl.orthogonalize(G)
    assert np.array_equal(impl.orthogonalize(-G), -O)
    assert np.array_equal(impl.orthogonalize(G.T), O.T)
    assert np.array_equal(impl.orthogonalize(8.0 * G), O)
    assert np.array_equal(impl.orthogonalize(2.0 ** -20 * G), O)
    p = r.permutation(7)
    q = r.permutation(11)
    assert rel(impl.orthogonalize(G[p][:, q]), O[p][:, q]) < 1e-13


def test_singular_value_band(impl):
    # critical points of g fix the band: g has a local max at x1 and a local
    # min at x2; once a normalized singular value has grown past ~1.6e-3, five
    # steps leave it in [g(x2), g(x1)] = [0.6818, 1.2024].  The page's
    # "0.7-1.3" is this band, rounded.
    a, b, c = QUINTIC
    disc = math.sqrt(9 * b * b - 20 * a * c)
    x1 = math.sqrt((-3 * b - disc) / (10 * c))
    x2 = math.sqrt((-3 * b + disc) / (10 * c))
    lo, hi = oracle.quintic_scalar(x2, 1), oracle.quintic_scalar(x1, 1)
    assert 0.68 < lo < 0.69 and 1.20 < hi < 1.21
    r = rng(21)
    m, n = 20, 30
    U, _ = np.linalg.qr(r.standard_normal((m, m)))
    V, _ = np.linalg.qr(r.standard_normal((n, n)))
    S = np.geomspace(1.0, 1e-2, m)
    assert (S / np.linalg.norm(S)).min() > 1.6e-3
    G = U @ np.diag(S) @ V[:, :m].T
    sv = np.linalg.svd(impl.orthogonalize(G), compute_uv=False)
    assert sv.max() <= hi + 1e-12 and sv.min() >= lo - 1e-12
    # below the threshold the map is ~ a^5 x: tiny singular values stay tiny
    S2 = np.concatenate([[1.0], np.full(m - 1, 1e-6)])
    G2 = U @ np.diag(S2) @ V[:, :m].T
    sv2 = np.sort(np.linalg.svd(impl.orthogonalize(G2), compute_uv=False))
    assert np.allclose(sv2[:-1], a ** 5 * 1e-6, rtol=1e-4)


def test_zero_and_empty(impl):
    assert np.array_equal(impl.orthogonalize(np.zeros((3, 4))), np.zeros((3, 4)))
    assert impl.orthogonalize(np.zeros((0, 4))).shape == (0, 4)
    with pytest.raises(ValueError):
        impl.orthogonalize(np.ones((2, 2)), method="bogus")
