"""Helpers of the GPU parity tests: run the HIP path through the C-ABI
binding and bring results back as float64 numpy arrays for the oracle."""
from __future__ import annotations

import numpy as np
import torch

import matrix_orthogonalizing_optimizer_amd as mo


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: the gpu tests need an MI355X")
    mo.lib()  # fail loudly when libmuon.so is missing
    return torch.device("cuda:0")


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def stored(x: np.ndarray, dtype) -> np.ndarray:
    """An fp64 oracle result rounded (RNE) to the storage dtype of the
    tensor it is compared with, back in fp64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(dtype).to(torch.float64).numpy()


def to_dev(x, dtype, device):
    return torch.as_tensor(np.asarray(x)).to(device=device, dtype=dtype).contiguous()


class StepRunner:
    """Owns plan + workspace for one shape table and runs muon_step."""

    def __init__(self, table, method=0, ns_dtype=-1, device=None):
        self.device = device or dev()
        self.table = table
        self.plan = mo.muon_plan_create(table, method, ns_dtype)
        nb = mo.muon_plan_workspace_bytes(self.plan)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=self.device)

    def step(self, params, grads, moms, eas, ess, hp, update_outs=None):
        mo.muon_step(self.plan, params, grads, moms, eas, ess, hp, self.ws, update_outs=update_outs)


def hp_from(d: dict, adam_step: int = 1, coeffs=None):
    return mo.make_hparams(lr=d["lr"], momentum=d["momentum"], weight_decay=d["weight_decay"],
                           nesterov=d["nesterov"], ns_steps=d["ns_steps"], coeffs=coeffs,
                           adam_lr=d["adam_lr"], adam_beta1=d["adam_beta1"],
                           adam_beta2=d["adam_beta2"], adam_eps=d["adam_eps"],
                           adam_weight_decay=d["adam_weight_decay"], adam_step=adam_step)


def block_rel_max(a, b, bs: int = 256) -> float:
    """Largest relative Frobenius error over the bs x bs blocks of a unit (the
    GEMM's output tile size): a single wrong output tile, which moves a large
    unit's overall error by only ~sqrt(tile / unit), shows here as O(1)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    worst = 0.0
    for i in range(0, b.shape[0], bs):
        for j in range(0, b.shape[1], bs):
            nb = np.linalg.norm(b[i:i + bs, j:j + bs])
            if nb == 0.0:
                continue
            worst = max(worst, float(np.linalg.norm(a[i:i + bs, j:j + bs] - b[i:i + bs, j:j + bs]) / nb))
    return worst


# Per-block bound next to the per-unit 2e-2 of the bf16 path: a block holds
# a small share of a unit's elements, so its error fluctuates more than the
# unit's; a tile that is wrong reads O(1).
BLOCK_TOL_BF16 = 5e-2
