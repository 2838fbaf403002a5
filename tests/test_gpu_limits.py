"""ns_orthogonalize on units at the library's addressing limit: an operand of
n x round_up(m, 8) elements just under 2^31 bytes (the planner rejects
larger ones), so every 32-bit buffer offset of the GEMMs and of the
transposing copy reaches its largest values.

The input is exactly rank one in the storage dtype (entries are products of
+-0.5, +-1, +-2), so its normalized singular value is 1 and the exact result
at any size is g5 * u v^T / (|u| |v|), g5 = g(g(g(g(g(1))))) for the quintic
g(x) = a x + b x^3 + c x^5 ("Newton-Schulz Iteration"; every step acts on the
single singular value).  Checked on every row of the unit at a sample of 512
columns.  Rounding errors of a step fall mostly in the directions of the zero
singular values, which the remaining quintic steps amplify by up to
a^5 ~ 485 (g'(0) = a), so the bounds are looser than the workload parity
bounds; an addressing error would be O(1).  fp32: ~1e-6 per step, amplified:
bound 1e-3 (measured 4.6e-4).  bf16: rounding P's diagonal (a = 3.4445) to
bf16 alone perturbs each step by ~0.2%, and the same chain emulated in numpy
on rank-one inputs of 256 x 8192, 1024 x 32768 and 512 x 65536 errs by
1.8-2.3e-2: bound 4e-2."""
import math

import pytest
import torch

mo = pytest.importorskip("matrix_orthogonalizing_optimizer_amd")

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)


def _g5():
    x = 1.0
    a, b, c = QUINTIC
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _pm(n, gen):
    vals = torch.tensor([0.5, -0.5, 1.0, -1.0, 2.0, -2.0], dtype=torch.float64)
    return vals[torch.randint(0, 6, (n,), generator=gen)]


@pytest.mark.parametrize("dtype,n,tall,tol", [
    (torch.bfloat16, 262136, False, 4e-2),
    (torch.bfloat16, 262136, True, 4e-2),
    (torch.float32, 131064, False, 1e-3),
])
def test_rank_one_at_addressing_limit(dtype, n, tall, tol):
    m = 4096
    es = 2 if dtype == torch.bfloat16 else 4
    assert n * m * es < 2 ** 31 <= (n + 8) * m * es  # within 8 of the largest n the planner accepts
    print(f"ns_orthogonalize rank-1 {'tall' if tall else 'wide'} {m}x{n} {dtype}", flush=True)
    gen = torch.Generator().manual_seed(n + (7 if tall else 0))
    u, v = _pm(m, gen), _pm(n, gen)
    d = torch.device("cuda:0")
    ud, vd = u.to(d, dtype), v.to(d, dtype)
    X = torch.outer(vd, ud) if tall else torch.outer(ud, vd)  # exact in both dtypes
    mo.ns_orthogonalize(X)
    torch.cuda.synchronize()
    cols = torch.randperm(n, generator=gen)[:512].to(d)
    got = (X[cols, :].t() if tall else X[:, cols]).double().cpu()
    expect = _g5() * torch.outer(u, v[cols.cpu()]) / (u.norm() * v.norm())
    e = float((got - expect).norm() / expect.norm())
    assert math.isfinite(e) and e <= tol, e
