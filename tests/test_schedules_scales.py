"""Coefficient schedules and update-scale modes: the library's schedule table
(host call, no GPU), and pins of both references' schedules and scales
against what the pages and the mathematics fix."""
import math

import numpy as np
import pytest

import oracle
from oracle import cref

QUINTIC = (3.4445, -4.7750, 2.0315)


@pytest.fixture(params=["numpy", "cpp"])
def impl(request):
    return oracle if request.param == "numpy" else cref


def _lib():
    mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")
    try:
        mo.lib()
    except Exception as e:  # library not built
        pytest.skip(str(e))
    return mo


def test_library_schedule_tables():
    mo = _lib()
    q = mo.muon_ns_coefficients(mo.MUON_COEFF_QUINTIC, 5)
    assert len(q) == 5 and all(np.allclose(r, QUINTIC, rtol=1e-7) for r in q)
    h = mo.muon_ns_coefficients(mo.MUON_COEFF_HYBRID, 10)
    assert all(np.allclose(r, QUINTIC, rtol=1e-7) for r in h[:8])
    assert h[8] == h[9] == (1.875, -1.25, 0.375)
    # the same tables as both references
    assert np.allclose(np.array(h), np.array(oracle.hybrid_schedule(10)), rtol=1e-7)
    assert np.allclose(np.array(h), np.array(cref.coefficients("hybrid", 10)), rtol=1e-7)
    with pytest.raises(mo.MuonError):
        mo.muon_ns_coefficients(mo.MUON_COEFF_HYBRID, 1)
    with pytest.raises(mo.MuonError):
        mo.muon_ns_coefficients(7, 5)


def test_refined_polynomial_conditions():
    # p(x) = a x + b x^3 + c x^5 with p(1) = 1, p'(1) = 0, p''(1) = 0: three
    # linear conditions whose unique solution is (15/8, -5/4, 3/8)
    M = np.array([[1.0, 1.0, 1.0], [1.0, 3.0, 5.0], [0.0, 6.0, 20.0]])
    a, b, c = np.linalg.solve(M, [1.0, 0.0, 0.0])
    assert np.allclose((a, b, c), oracle.REFINED, atol=1e-15)
    # it maps the quintic's band into a neighbourhood of 1 twice as tightly
    p = lambda x: a * x + b * x ** 3 + c * x ** 5
    for x in np.linspace(0.6818, 1.2024, 50):
        assert abs(p(p(x)) - 1.0) < 5e-3


def closed_form(G, sched):
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = np.linalg.norm(G)
    mapped = np.array([oracle.quintic_scalar(x / s, len(sched), sched) for x in S])
    return (U * mapped) @ Vt


@pytest.mark.parametrize("shape", [(12, 30), (30, 12)])
def test_hybrid_ten_steps_closed_form(shape, impl):
    G = np.random.default_rng(shape[0]).standard_normal(shape)
    sched = oracle.hybrid_schedule(10)
    O = impl.orthogonalize(G, steps=10, coeffs=sched)
    assert np.linalg.norm(O - closed_form(G, sched)) / np.linalg.norm(O) < 1e-12
    # singular values of normalized size >= ~1e-3 end within 5e-3 of 1
    sv = np.linalg.svd(O, compute_uv=False)
    assert np.max(np.abs(sv - 1.0)) < 5e-3


@pytest.mark.parametrize("rows,cols,moon,spec,unit", [
    (4096, 14336, 23.9466, 0.534522, 119.7330), (14336, 4096, 23.9466, 1.870829, 119.7330),
    (768, 768, 5.5426, 1.0, 27.7128), (128, 2048, 9.0510, 0.25, 45.2548)])
def test_scale_modes(rows, cols, moon, spec, unit, impl):
    assert impl.muon_scale(rows, cols) == pytest.approx(moon, abs=5e-5)
    assert impl.muon_scale(rows, cols, mode="spectral") == pytest.approx(spec, abs=5e-6)
    assert impl.muon_scale(rows, cols, mode="unit_rms") == pytest.approx(unit, abs=5e-5)
    # gamma multiplies every mode; scale_dim replaces max(A, B) where it is used
    assert impl.muon_scale(rows, cols, mode="unit_rms", gamma=0.25) == pytest.approx(unit / 4, abs=2e-5)
    assert impl.muon_scale(rows, cols, scale_dim=100, mode="unit_rms") == pytest.approx(10.0)
    assert impl.muon_scale(rows, cols, scale_dim=100, mode="spectral") == pytest.approx(spec, abs=5e-6)
    with pytest.raises(ValueError):
        impl.muon_scale(rows, cols, mode="bogus")


def test_unit_rms_scale_gives_unit_rms_update(impl):
    # with O semi-orthogonal, ||O||_F^2 = min(m, n), so sqrt(max(m, n)) O has
    # RMS 1 ([Blog] DeepSeek-V4 listing: "Rescale update RMS")
    r = np.random.default_rng(3)
    for shape in [(8, 20), (20, 8)]:
        G = r.standard_normal(shape)
        U, _, Vt = np.linalg.svd(G, full_matrices=False)
        O = U @ Vt
        s = impl.muon_scale(*shape, mode="unit_rms")
        assert math.isclose(float(np.sqrt(np.mean((s * O) ** 2))), 1.0, rel_tol=1e-12)
