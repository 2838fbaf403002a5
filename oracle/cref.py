"""ctypes binding of the plain C++ fp64 reference (oracle/muon_ref.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: loaded by the test
suite, the smoke check and the benchmark's CPU-baseline leg, never by the
product path.  ``build()`` compiles the library with g++ (no GPU, no HIP)."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "muon_ref.cpp")
LIB = os.path.join(HERE, "libmuonref.so")

_lib = None
_D = ctypes.POINTER(ctypes.c_double)


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-Wall", SRC, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        L.ref_set_threads.argtypes = [ctypes.c_int32]
        L.ref_threads.restype = ctypes.c_int32
        L.ref_momentum.argtypes = [_D, _D, ctypes.c_int64, ctypes.c_double, ctypes.c_int32, _D]
        L.ref_orthogonalize.argtypes = [_D, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _D,
                                        ctypes.c_int32, _D]
        L.ref_orthogonalize.restype = ctypes.c_int32
        L.ref_muon_scale.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double]
        L.ref_muon_scale.restype = ctypes.c_double
        L.ref_muon_scale_mode.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                          ctypes.c_int32, ctypes.c_double]
        L.ref_muon_scale_mode.restype = ctypes.c_double
        L.ref_coefficients.argtypes = [ctypes.c_int32, ctypes.c_int32, _D]
        L.ref_coefficients.restype = ctypes.c_int32
        L.ref_weight_update.argtypes = [_D, _D, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_double]
        L.ref_adamw.argtypes = [_D, _D, _D, _D, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double]
        L.ref_plan.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                               ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                               ctypes.POINTER(ctypes.c_int32)]
        L.ref_plan.restype = ctypes.c_int64
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def set_threads(n: int) -> None:
    lib().ref_set_threads(int(n))


def threads() -> int:
    return int(lib().ref_threads())


def momentum(M, G, mu: float, nesterov: bool):
    """Returns (M_new, U)."""
    M = _f64(M).copy()
    G = _f64(G)
    U = np.empty_like(M)
    lib().ref_momentum(_p(M), _p(G), M.size, mu, 1 if nesterov else 0, _p(U))
    return M, U


def orthogonalize(G, steps: int = 5, coeffs: Optional[Sequence] = None, method: str = "standard"):
    G = _f64(G)
    rows, cols = G.shape
    c = None
    if coeffs is not None:
        c = _f64(coeffs)
        if c.shape == (3,):
            c = np.tile(c, (steps, 1))
        if c.shape != (steps, 3):
            raise ValueError("coeffs must be (3,) or (steps, 3)")
        c = np.ascontiguousarray(c)
    if method not in ("standard", "gram", "gram_restart"):
        raise ValueError(f"unknown ns method {method!r}")
    O = np.empty_like(G)
    st = lib().ref_orthogonalize(_p(G), rows, cols, steps, _p(c) if c is not None else None,
                                 {"standard": 0, "gram": 1, "gram_restart": 3}[method], _p(O))
    if st != 0:
        raise ValueError("ref_orthogonalize rejected its arguments")
    return O


_MODES = {"moonlight": 0, "spectral": 1, "unit_rms": 2}


def muon_scale(rows: int, cols: int, scale_dim: int = 0, rms_scale: float = 0.2, mode: str = "moonlight",
               gamma: float = 1.0) -> float:
    if mode not in _MODES:
        raise ValueError(f"unknown scale mode {mode!r}")
    return float(lib().ref_muon_scale_mode(rows, cols, scale_dim, rms_scale, _MODES[mode], gamma))


def coefficients(kind: str, steps: int):
    """steps x 3 schedule: "quintic" or "hybrid" (steps >= 2)."""
    out = np.zeros((max(steps, 1), 3))
    if lib().ref_coefficients({"quintic": 0, "hybrid": 1}[kind], steps, _p(out)) != 0:
        raise ValueError("bad schedule")
    return [tuple(r) for r in out[:steps].tolist()]


def weight_update(W, O, lr: float, wd: float, scale: float):
    W = _f64(W).copy()
    O = _f64(O)
    lib().ref_weight_update(_p(W), _p(O), W.size, lr, wd, scale)
    return W


def adamw(W, g, m, v, t: int, lr: float, b1: float, b2: float, eps: float, wd: float):
    W, m, v = _f64(W).copy(), _f64(m).copy(), _f64(v).copy()
    g = _f64(g)
    lib().ref_adamw(_p(W), _p(g), _p(m), _p(v), W.size, t, lr, b1, b2, eps, wd)
    return W, m, v


def plan(table, method: int = 0, ns_dtype: int = -1):
    """(units: list of 6-tuples, buckets: list of 8-tuples), both bucket-ordered."""
    t = np.ascontiguousarray(np.asarray(table, dtype=np.int64).reshape(-1, 6))
    cap = int(sum(max(1, r[2] // r[4]) if r[4] > 0 else 1 for r in t.tolist())) + 1
    units = np.zeros((cap, 6), dtype=np.int64)
    buckets = np.zeros((cap, 8), dtype=np.int32)
    nb = ctypes.c_int32(0)
    nu = lib().ref_plan(t.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(t), method, ns_dtype,
                        units.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), cap,
                        buckets.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap, ctypes.byref(nb))
    if nu < 0:
        raise RuntimeError("ref_plan capacity")
    return [tuple(u) for u in units[:nu].tolist()], [tuple(b) for b in buckets[:nb.value].tolist()]


# the numpy reference's names, so tests can run the same pins on both
momentum_update = momentum
adamw_update = adamw


class Unit(tuple):
    """(param, row0, rows, cols, tall, scale_dim) of one unit, with names."""
    __slots__ = ()
    param = property(lambda self: self[0])
    row0 = property(lambda self: self[1])
    rows = property(lambda self: self[2])
    cols = property(lambda self: self[3])
    tall = property(lambda self: bool(self[4]))
    scale_dim = property(lambda self: self[5])


def units_in_table_order(table):
    """The C++ planner's units, listed parameter by parameter (row blocks in
    ascending order) instead of bucket by bucket."""
    units, _ = plan(table, 0, -1)
    return [Unit(u) for u in sorted(units, key=lambda u: (u[0], u[1]))]


def muon_step(table, params, grads, moms, exp_avgs, exp_avg_sqs, hp, method: str = "standard",
              units_subset=None, want_updates: bool = False, adamw_params: bool = True):
    """One optimizer step over a shape table with the C++ reference's
    functions only (this is glue: every arithmetic step runs in
    muon_ref.cpp).  Same arguments and result as the numpy reference's
    ``muon_step``: ``hp`` carries lr, momentum, weight_decay, nesterov,
    ns_steps, coeffs, rms_scale, scale_mode, extra_scale and the adam_*
    fields; units are numbered in table order.  ``units_subset`` restricts
    the Muon work to those units, and then only the parameters they touch
    are copied (the others may be passed as None and come back as None);
    ``adamw_params=False`` leaves the AdamW parameters out."""
    units = units_in_table_order(table)
    sel = list(range(len(units)) if units_subset is None else units_subset)
    touched = {units[ui].param for ui in sel}
    if adamw_params:
        touched |= {p for p, row in enumerate(table) if row[0] == 1}
    cp = lambda xs, p: None if xs[p] is None or p not in touched else _f64(xs[p]).copy()
    W_out = [cp(params, p) for p in range(len(table))]
    M_out = [cp(moms, p) for p in range(len(table))]
    ea_out = [cp(exp_avgs, p) for p in range(len(table))]
    es_out = [cp(exp_avg_sqs, p) for p in range(len(table))]
    updates = {}
    for ui in sel:
        u = units[ui]
        r0, r1 = u.row0, u.row0 + u.rows
        M_new, U = momentum(_f64(moms[u.param])[r0:r1], _f64(grads[u.param])[r0:r1], hp.momentum,
                            hp.nesterov)
        M_out[u.param][r0:r1] = M_new
        O = orthogonalize(U, hp.ns_steps, hp.coeffs, method)
        scale = muon_scale(u.rows, u.cols, u.scale_dim, hp.rms_scale, hp.scale_mode, hp.extra_scale)
        W_out[u.param][r0:r1] = weight_update(_f64(params[u.param])[r0:r1], O, hp.lr, hp.weight_decay,
                                              scale)
        if want_updates:
            updates[ui] = O
    for p, row in enumerate(table):
        if row[0] != 1 or not adamw_params:
            continue
        W_out[p], ea_out[p], es_out[p] = adamw(params[p], grads[p], exp_avgs[p], exp_avg_sqs[p],
                                               hp.adam_step, hp.adam_lr, hp.adam_beta1, hp.adam_beta2,
                                               hp.adam_eps, hp.adam_weight_decay)
    return {"W": W_out, "M": M_out, "exp_avg": ea_out, "exp_avg_sq": es_out, "O": updates,
            "units": units}
