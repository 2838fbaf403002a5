"""Seeded synthetic inputs shared by the oracle and the GPU path.

Holds none of the method's arithmetic.  The gradient generator follows the
workload description: a rank-r sum of outer products of Gaussian unit vectors
with singular values geometric from 1 down to 1e-3, plus iid Gaussian noise of
element standard deviation 1e-3 (1e-3 relative to the top singular value).
Weights are N(0, 0.02^2); AdamW gradients N(0, 1e-6).

All draws come from torch generators seeded per (workload, parameter, step),
on the device the caller names: CPU for small cases, the GPU for full-size
workloads (then sampled units are copied back for the oracle, so both sides
always see the same bytes).
"""
from __future__ import annotations

import torch

NOISE_STD = 1e-3
W_STD = 0.02
ADAM_G_STD = 1e-3


def stream_seed(base: int, *ids: int) -> int:
    """Deterministic 63-bit seed for one (workload, param, step, ...) stream."""
    h = (base * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019) & 0xFFFFFFFFFFFFFFFF
    for i in ids:
        h ^= (i + 0x9E3779B97F4A7C15 + (h << 6) + (h >> 2)) & 0xFFFFFFFFFFFFFFFF
        h = (h * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def lowrank_gradient(rows: int, cols: int, rank: int, seed: int, device="cpu",
                     dtype=torch.float32, noise_std: float = NOISE_STD) -> torch.Tensor:
    """G = sum_i s_i u_i v_i^T + E with s_i = 10^(-3 (i-1)/(r-1)), u_i, v_i
    Gaussian unit vectors (not orthogonalized), E iid N(0, noise_std^2).
    Computed in fp32 (fp64 on CPU) then stored in ``dtype``."""
    g = _gen(device, seed)
    wdt = torch.float64 if str(device) == "cpu" else torch.float32
    r = max(1, min(rank, rows, cols))
    if r > 1:
        s = torch.tensor([10.0 ** (-3.0 * i / (r - 1)) for i in range(r)], dtype=wdt, device=device)
    else:
        s = torch.ones(1, dtype=wdt, device=device)
    U = torch.randn(rows, r, generator=g, device=device, dtype=wdt)
    U = U / U.norm(dim=0, keepdim=True)
    V = torch.randn(cols, r, generator=g, device=device, dtype=wdt)
    V = V / V.norm(dim=0, keepdim=True)
    G = (U * s) @ V.T
    G += noise_std * torch.randn(rows, cols, generator=g, device=device, dtype=wdt)
    return G.to(dtype)


def conditioned_matrix(rows: int, cols: int, smin: float, smax: float, seed: int, device="cpu",
                       dtype=torch.float32) -> torch.Tensor:
    """U diag(s) V^T with U, V random orthonormal (QR of Gaussian matrices)
    and the min(rows, cols) singular values s uniform in [smin, smax]: a
    well-conditioned input whose normalized singular values all stay clear of
    the range the quintic amplifies.  Computed in fp64 on the CPU."""
    g = _gen("cpu", seed)
    k = min(rows, cols)
    U, _ = torch.linalg.qr(torch.randn(rows, k, generator=g, dtype=torch.float64))
    V, _ = torch.linalg.qr(torch.randn(cols, k, generator=g, dtype=torch.float64))
    s = smin + (smax - smin) * torch.rand(k, generator=g, dtype=torch.float64)
    return ((U * s) @ V.T).to(device=device, dtype=dtype)


def normal(rows: int, cols: int, std: float, seed: int, device="cpu", dtype=torch.float32):
    g = _gen(device, seed)
    wdt = torch.float64 if str(device) == "cpu" else torch.float32
    x = torch.randn(rows, cols, generator=g, device=device, dtype=wdt) * std
    return x.to(dtype)


def torch_dtype(code: int):
    return torch.float32 if code == 0 else torch.bfloat16


def make_state(workload, device="cpu", base_seed: int = 0, wl_id: int = 0):
    """Parameters, zero momentum / AdamW moments for a workload's table."""
    params, moms, ea, es = [], [], [], []
    for p, (kind, dt, rows, cols, _s, _sd) in enumerate(workload.table):
        tdt = torch_dtype(dt)
        params.append(normal(rows, cols, W_STD, stream_seed(base_seed, wl_id, p, 1 << 20),
                             device, tdt))
        if kind == 0:
            moms.append(torch.zeros(rows, cols, dtype=torch.float32, device=device))
            ea.append(None)
            es.append(None)
        else:
            moms.append(None)
            ea.append(torch.zeros(rows, cols, dtype=torch.float32, device=device))
            es.append(torch.zeros(rows, cols, dtype=torch.float32, device=device))
    return params, moms, ea, es


def make_grads(workload, step: int, device="cpu", base_seed: int = 0, wl_id: int = 0):
    """Fresh gradients for one step (a split parameter draws one gradient for
    the whole parent weight, then is split)."""
    grads = []
    for p, (kind, dt, rows, cols, _s, _sd) in enumerate(workload.table):
        seed = stream_seed(base_seed, wl_id, p, step)
        tdt = torch_dtype(dt)
        if kind == 0:
            grads.append(lowrank_gradient(rows, cols, workload.rank, seed, device, tdt))
        else:
            grads.append(normal(rows, cols, ADAM_G_STD, seed, device, tdt))
    return grads
