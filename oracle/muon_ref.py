"""Plain fp64 CPU reference of the Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, helpers or constants); the two meet only through the
seeded input generators in ``workloads``.

Every function is written from the pages in the order and notation they use,
in float64, with numpy's matmul as the only library primitive.  There is no
blocking, fusion or reordering beyond what the cited passage states.

Sources (web pages; cited by title and section):
  [Blog]      "Muon Optimizer and the Distributed Implementation" (blog.chensy.moe)
  [Moonlight] the Kimi/Moonlight summary page ("...Muon优化器可替代 AdamW..."),
              sections "权重衰减机制", "参数更新尺度调整:一致的更新 RMS" and "代码"
              (the PyTorch ``Muon`` class printed there)
  [DeepSpeed] "DeepSpeed 集成 Muon 优化器实战..." (NS_METHODS, Gram variant)
  [MindSpeed] the MindSpeed "Muon 优化器" document (QKV split, 实现原理)

Readings taken where the pages are silent or garbled are listed in the
project's design notes; each function below states the one it relies on.

Parity pins: every function here is pinned by tests against closed forms,
hand-reduced cases, invariants or brute force (see tests/test_oracle_*.py).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

# [Blog] "Newton-Schulz Iteration": the quintic coefficients found by gradient
# descent, used five times ("NewtonSchulz5").
QUINTIC = (3.4445, -4.7750, 2.0315)
DEFAULT_STEPS = 5
# [Moonlight] "参数更新尺度调整": update RMS matched with the constant 0.2.
RMS_SCALE = 0.2


# [Blog] DeepSeek-V4 listing: "HybridNewtonSchulz" runs ten steps, eight with
# the quintic and the last two with an improved Newton iteration that brings
# the singular values closer to 1.  Its coefficients are not printed; the
# reading taken is the odd quintic p with p(1) = 1, p'(1) = p''(1) = 0, the
# second-order expansion of x (x^2)^(-1/2) around 1 ([Blog] "Sign of a Matrix").
REFINED = (15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0)


def hybrid_schedule(steps: int) -> List[Tuple[float, float, float]]:
    """steps - 2 quintic steps, then two refining steps (steps >= 2)."""
    if steps < 2:
        raise ValueError("the hybrid schedule needs at least two steps")
    return [QUINTIC] * (steps - 2) + [REFINED] * 2


def coeff_schedule(steps: int, coeffs: Optional[Sequence] = None) -> List[Tuple[float, float, float]]:
    """Per-step (a, b, c).  ``coeffs`` is None (the quintic every step), one
    triple (used every step) or a list of ``steps`` triples."""
    if coeffs is None:
        return [QUINTIC] * steps
    arr = np.asarray(coeffs, dtype=np.float64)
    if arr.shape == (3,):
        return [tuple(float(x) for x in arr)] * steps
    if arr.shape != (steps, 3):
        raise ValueError(f"coeffs must be (3,) or ({steps}, 3), got {arr.shape}")
    return [tuple(float(x) for x in row) for row in arr]


# --------------------------------------------------------------------------
# Momentum  ([Blog] "Formulation of Muon Optimizer"; [Moonlight] "代码", step)
# --------------------------------------------------------------------------

def momentum_update(M: np.ndarray, G: np.ndarray, mu: float, nesterov: bool):
    """M_t = mu*M_{t-1} + G_t; the matrix to orthogonalize is G_t + mu*M_t
    with Nesterov ([Blog] "Variation of Muon Optimizer": msign(beta*M_t + G_t);
    the [Moonlight] "代码" section's step does the same: the buffer is
    scaled by the momentum and the gradient added, then the gradient plus
    the momentum times the buffer is orthogonalized), else M_t itself.
    Returns (M_t, U)."""
    M = np.asarray(M, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M_new = mu * M + G
    U = G + mu * M_new if nesterov else M_new.copy()
    return M_new, U


# --------------------------------------------------------------------------
# Orthogonalization  ([Blog] "Orthogonalization of Gradients",
# "Sign of a Matrix", "Newton-Schulz Iteration")
# --------------------------------------------------------------------------

def frobenius_normalize(X: np.ndarray):
    """X / ||X||_F, which puts every singular value in [0, 1] ([Blog]
    "Newton-Schulz Iteration", first added condition).  The page prints no
    epsilon; the one reading taken is that a zero matrix stays zero (its
    orthogonalized update is then zero).  Returns (X_normalized, s)."""
    X = np.asarray(X, dtype=np.float64)
    s = math.sqrt(float(np.sum(X * X)))
    if s == 0.0:
        return np.zeros_like(X), 0.0
    return X / s, s


def ns_standard(X: np.ndarray, schedule) -> np.ndarray:
    """Newton-Schulz on a normalized X with rows <= cols.  Each step applies
    phi(X) = (a + b X X^T + c (X X^T)^2) X ([Blog] "Newton-Schulz Iteration"),
    evaluated in Horner form a X + (b A + c A A) X with A = X X^T, as the page
    says implementations do."""
    X = np.asarray(X, dtype=np.float64)
    for a, b, c in schedule:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def ns_gram(X: np.ndarray, schedule, restart_after: int = 0, dtype=np.float64) -> np.ndarray:
    """Gram variant ([DeepSpeed]: iterate on the small square Gram matrix
    R = X X^T instead of the rectangular X).  The page describes only that;
    the reading taken is the exact-arithmetic rewrite of ``ns_standard``:
    with P_k = a I + b R_k + c R_k^2 one has X_{k+1} = P_k X_k, so
    R_{k+1} = P_k R_k P_k and X_N = (P_{N-1} ... P_0) X_0 = Q X_0.

    ``restart_after`` = r > 0 restarts the chain once, after r steps (an
    extension; the pages describe no restart): X_r = Q X_0 is formed, R is
    recomputed as X_r X_r^T and Q starts again from I, so the result is
    Q' X_r.  In exact arithmetic that changes nothing; in rounded arithmetic
    the chain's error restarts from the rectangular iterate.  ``dtype``: the
    arithmetic of the chain (fp64; a pin rounds it to fp32 to see the
    restart)."""
    X = np.asarray(X, dtype=np.float64).astype(dtype)
    m = X.shape[0]
    I = np.eye(m, dtype=dtype)
    R = X @ X.T
    Q = I.copy()
    steps = len(schedule)
    for k, (a, b, c) in enumerate(schedule):
        a, b, c = dtype(a), dtype(b), dtype(c)
        P = a * I + b * R + c * (R @ R)
        Q = P @ Q
        if k < steps - 1:
            if restart_after > 0 and k + 1 == restart_after:
                X = Q @ X
                R = X @ X.T
                Q = I.copy()
            else:
                R = P @ R @ P
    return (Q @ X).astype(np.float64)


def restart_step(steps: int) -> int:
    """Where the restarted Gram chain restarts: after ceil(steps / 2) steps
    when there are at least two (the reading taken for the extension)."""
    return (steps + 1) // 2 if steps >= 2 else 0


def orthogonalize(G: np.ndarray, steps: int = DEFAULT_STEPS, coeffs=None,
                  method: str = "standard") -> np.ndarray:
    """NewtonSchulz(G) for one logically independent matrix G (rows x cols).

    A tall G is processed as its transpose: msign(G) = (G G^T)^{-1/2} G =
    G (G^T G)^{-1/2} ([Blog] "Sign of a Matrix", first theorem), so the
    iteration may run on whichever Gram side is smaller and the result is
    transposed back.  Then Frobenius-normalize and iterate."""
    G = np.asarray(G, dtype=np.float64)
    if G.ndim != 2:
        raise ValueError("orthogonalize expects a 2-D matrix")
    rows, cols = G.shape
    if rows == 0 or cols == 0:
        return np.zeros_like(G)
    tall = rows > cols
    X = G.T if tall else G
    X, s = frobenius_normalize(X)
    if s == 0.0:
        return np.zeros_like(G)
    sched = coeff_schedule(steps, coeffs)
    if method == "standard":
        X = ns_standard(X, sched)
    elif method == "gram":
        X = ns_gram(X, sched)
    elif method == "gram_restart":
        X = ns_gram(X, sched, restart_after=restart_step(len(sched)))
    else:
        raise ValueError(f"unknown ns method {method!r}")
    return X.T.copy() if tall else X


def quintic_scalar(x: float, steps: int = DEFAULT_STEPS, coeffs=None) -> float:
    """The scalar map each singular value undergoes: g(x) = a x + b x^3 + c x^5
    applied ``steps`` times ([Blog] "Newton-Schulz Iteration": phi(G) =
    U (a S + b S^3 + c S^5) V^T).  Used by closed-form checks."""
    for a, b, c in coeff_schedule(steps, coeffs):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


# --------------------------------------------------------------------------
# Update  ([Moonlight] "权重衰减机制", "参数更新尺度调整", "代码")
# --------------------------------------------------------------------------

def muon_scale(rows: int, cols: int, scale_dim: int = 0, rms_scale: float = RMS_SCALE,
               mode: str = "moonlight", gamma: float = 1.0) -> float:
    """Scale of the orthogonalized update of a rows x cols unit (d_out x d_in).
    "moonlight": 0.2 * sqrt(max(A, B)) ([Moonlight] "参数更新尺度调整"; the
    code's ``adjust_lr_for_muon``); "spectral": sqrt(d_out / d_in) ([Blog]
    "Variation of Muon Optimizer", the muP form from dualizing under the
    RMS->RMS norm); "unit_rms": sqrt(max(n, m)) ([Blog] DeepSeek-V4 listing,
    "Rescale update RMS").  Each is multiplied by gamma, the listing's update
    rescaling factor.  For a split block the reading taken is the block's own
    shape (the listing rescales each logically independent weight);
    ``scale_dim`` > 0 overrides max(A, B)."""
    d = scale_dim if scale_dim > 0 else max(rows, cols)
    if mode == "moonlight":
        s = rms_scale * math.sqrt(d)
    elif mode == "spectral":
        s = math.sqrt(rows / cols)
    elif mode == "unit_rms":
        s = math.sqrt(d)
    else:
        raise ValueError(f"unknown scale mode {mode!r}")
    return gamma * s


def weight_update(W: np.ndarray, O: np.ndarray, lr: float, wd: float, scale: float) -> np.ndarray:
    """W_t = W_{t-1} - lr * (scale * O_t + wd * W_{t-1}) ([Moonlight]
    "参数更新尺度调整" update formula; "权重衰减机制": decoupled weight
    decay), i.e. W_{t-1} (1 - lr wd) - lr scale O_t."""
    W = np.asarray(W, dtype=np.float64)
    return W * (1.0 - lr * wd) - (lr * scale) * np.asarray(O, dtype=np.float64)


def adamw_update(W, g, m, v, t: int, lr: float, beta1: float, beta2: float,
                 eps: float, wd: float):
    """The AdamW fallback for the parameters Muon does not take ([Moonlight]
    "代码": the optimizer's AdamW backup), at step t >= 1, as mathematics:
        m_t = beta1 m_{t-1} + (1 - beta1) g
        v_t = beta2 v_{t-1} + (1 - beta2) g^2
        W_t = W_{t-1} (1 - lr wd)
              - lr sqrt(1 - beta2^t) / (1 - beta1^t) * m_t / (eps + sqrt(v_t))
    The bias corrections multiply the step, so eps is added to the
    uncorrected sqrt(v_t) (the page's placement; it differs from textbook
    AdamW by eps sqrt(1 - beta2^t)).  Returns (W_t, m_t, v_t)."""
    W = np.asarray(W, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m_t = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_t = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    step = lr * math.sqrt(1.0 - beta2 ** t) / (1.0 - beta1 ** t)
    W_t = W * (1.0 - lr * wd) - step * (m_t / (eps + np.sqrt(v_t)))
    return W_t, m_t, v_t


# --------------------------------------------------------------------------
# Shape table -> units -> buckets  (independent brute-force planner)
# --------------------------------------------------------------------------

KIND_MUON = 0
KIND_ADAMW = 1
DT_F32 = 0
DT_BF16 = 1


@dataclass
class OracleUnit:
    param: int
    row0: int
    rows: int
    cols: int
    scale_dim: int

    @property
    def tall(self) -> bool:
        return self.rows > self.cols

    @property
    def m(self) -> int:
        return min(self.rows, self.cols)

    @property
    def n(self) -> int:
        return max(self.rows, self.cols)


def plan_units(table) -> List[OracleUnit]:
    """Split each Muon parameter into its independent units, in table order.
    A parameter with split_rows > 0 is cut into consecutive row blocks of that
    height, each orthogonalized on its own ([MindSpeed] "QKV split": the fused
    QKV weight is split into Q/K/V sub-matrices, each orthogonalized, then put
    back; [DeepSpeed] per-attention-head "Muon Split")."""
    units = []
    for p, row in enumerate(table):
        kind, dtype, rows, cols, split_rows, scale_dim = row
        if kind != KIND_MUON or rows == 0 or cols == 0:
            continue
        h = split_rows if split_rows > 0 else rows
        r = 0
        while r < rows:
            units.append(OracleUnit(p, r, h, cols, scale_dim))
            r += h
    return units


def gram_fp16_ok(m: int, n: int) -> bool:
    """Where the Gram variant's power-of-two scaled fp16 chain stays within
    the bf16 tolerance on the workload gradients: m >= 512 and n >= 3 m
    (a rounding emulation of that chain gave 5.3e-2 at 512 x 860, 5.8e-2 at
    768 x 768 and 3.5e-2 at 256 x 512, at most 1.25e-2 inside).  The pages
    give no rule; this is the reading taken."""
    return m >= 512 and n >= 3 * m


def resolve_method(method: int, dt: int, m: int, n: int) -> int:
    """Method 2 ("auto") picks, per unit, the Gram variant where its fp16
    chain is accurate (``gram_fp16_ok``), which also lies where it executes
    less work than the standard method (standard: steps (3 m^2 n + m^3) with
    symmetric products, Gram: 3 m^2 n + (6 steps - 5) m^3, i.e. n/m > 5/3);
    the standard method otherwise.  An explicit Gram request (1) for the
    fp32 compute dtype (code 0) outside that region is served by the
    standard method: the fp32 Gram chain there measured above the fp32
    tolerance (1.1-1.8e-4 on 768 x 768, 512 x 860, 96 x 300).  The
    restarted Gram chain (3) is kept for the 16-bit compute dtype when
    m >= 256 (there its restart keeps the fp16 chain within the bf16
    tolerance) and resolved as a Gram request (1) otherwise."""
    if method == 2:
        return 1 if gram_fp16_ok(m, n) else 0
    if method == 3 and (dt == DT_F32 or m < 256):
        method = 1
    if method == 1 and dt == DT_F32 and not gram_fp16_ok(m, n):
        return 0
    return method


def resolve_compute_dtype(dt: int, method: int, m: int, n: int) -> int:
    """A bf16 (code 1) Gram unit outside ``gram_fp16_ok`` computes in fp32
    (code 0), so that an explicit request for the Gram variant never leaves
    the tolerance."""
    if method == 1 and dt == DT_BF16 and not gram_fp16_ok(m, n):
        return DT_F32
    return dt


def plan_buckets(table, method: int, ns_dtype: int = -1):
    """Group units with the same (m, n, tall, parameter dtype, compute dtype,
    method), the compute dtype as ``resolve_compute_dtype`` sets it.  Buckets are numbered by first appearance; units inside a bucket
    keep table order.  Brute force: for every unit, scan the buckets seen so
    far.  ``ns_dtype`` -1 means the compute dtype follows the parameter
    dtype."""
    units = plan_units(table)
    keys = []
    members = []
    for ui, u in enumerate(units):
        pdt = table[u.param][1]
        req = pdt if ns_dtype < 0 else ns_dtype
        meth = resolve_method(method, req, u.m, u.n)
        dt = resolve_compute_dtype(req, meth, u.m, u.n)
        key = (u.m, u.n, 1 if u.tall else 0, pdt, dt, meth)
        found = -1
        for bi, k in enumerate(keys):
            if k == key:
                found = bi
                break
        if found < 0:
            keys.append(key)
            members.append([ui])
        else:
            members[found].append(ui)
    return units, keys, members


# --------------------------------------------------------------------------
# Whole step over a shape table
# --------------------------------------------------------------------------

@dataclass
class OracleHparams:
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    nesterov: bool = True
    ns_steps: int = DEFAULT_STEPS
    coeffs: Optional[Sequence] = None
    rms_scale: float = RMS_SCALE
    adam_lr: float = 3e-4
    adam_beta1: float = 0.9
    adam_beta2: float = 0.95
    adam_eps: float = 1e-8
    adam_weight_decay: float = 0.1
    adam_step: int = 1
    scale_mode: str = "moonlight"
    extra_scale: float = 1.0


def muon_step(table, params, grads, moms, exp_avgs, exp_avg_sqs, hp: OracleHparams,
              method: str = "standard", units_subset: Optional[Sequence[int]] = None,
              want_updates: bool = False):
    """One optimizer step over a shape table (lists of fp64 arrays, updated
    copies returned).  Muon parameters follow [Moonlight] "代码" step():
    momentum, orthogonalize (per unit), weight decay then the scaled update;
    the rest take the AdamW fallback.  ``units_subset`` restricts the Muon work
    to those unit indices (the momentum of a parameter is updated only on the
    rows of the selected units).  Returns dict with W, M, m, v lists and, if
    asked, the per-unit orthogonalized update O."""
    units = plan_units(table)
    sel = range(len(units)) if units_subset is None else units_subset
    W_out = [None if p is None else np.array(p, dtype=np.float64) for p in params]
    M_out = [None if mm is None else np.array(mm, dtype=np.float64) for mm in moms]
    ea_out = [None if x is None else np.array(x, dtype=np.float64) for x in exp_avgs]
    es_out = [None if x is None else np.array(x, dtype=np.float64) for x in exp_avg_sqs]
    updates = {}
    for ui in sel:
        u = units[ui]
        r0, r1 = u.row0, u.row0 + u.rows
        G = np.asarray(grads[u.param], dtype=np.float64)[r0:r1]
        M = np.asarray(moms[u.param], dtype=np.float64)[r0:r1]
        M_new, U = momentum_update(M, G, hp.momentum, hp.nesterov)
        M_out[u.param][r0:r1] = M_new
        O = orthogonalize(U, hp.ns_steps, hp.coeffs, method)
        scale = muon_scale(u.rows, u.cols, u.scale_dim, hp.rms_scale, hp.scale_mode, hp.extra_scale)
        W = np.asarray(params[u.param], dtype=np.float64)[r0:r1]
        W_out[u.param][r0:r1] = weight_update(W, O, hp.lr, hp.weight_decay, scale)
        if want_updates:
            updates[ui] = O
    for p, row in enumerate(table):
        if row[0] != KIND_ADAMW:
            continue
        W, m, v = adamw_update(params[p], grads[p], exp_avgs[p], exp_avg_sqs[p],
                               hp.adam_step, hp.adam_lr, hp.adam_beta1, hp.adam_beta2,
                               hp.adam_eps, hp.adam_weight_decay)
        W_out[p], ea_out[p], es_out[p] = W, m, v
    return {"W": W_out, "M": M_out, "exp_avg": ea_out, "exp_avg_sq": es_out,
            "O": updates, "units": units}
