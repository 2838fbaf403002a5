"""Shape tables of the five synthetic Muon workloads.

A shape-table row is (kind, dtype, rows, cols, split_rows, scale_dim):
  kind       0 = Muon (2-D hidden weight), 1 = AdamW fallback (anything else)
  dtype      0 = fp32, 1 = bf16 (parameter and gradient storage)
  rows, cols the 2-D view of the parameter (vectors are 1 x len)
  split_rows 0 = one unit; h > 0 = independent row blocks of height h
  scale_dim  0 = the unit's max(rows, cols) in 0.2*sqrt(max(A, B)); else override

Holds no arithmetic of the method: it only describes the workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

MUON, ADAMW = 0, 1
F32, BF16 = 0, 1

Row = Tuple[int, int, int, int, int, int]


def _hp(**kw):
    base = dict(lr=0.02, momentum=0.95, weight_decay=0.1, nesterov=True, ns_steps=5,
                adam_lr=3e-4, adam_beta1=0.9, adam_beta2=0.95, adam_eps=1e-8,
                adam_weight_decay=0.1)
    base.update(kw)
    return base


@dataclass
class Workload:
    name: str
    table: List[Row]
    names: List[str]
    rank: int                 # rank of the synthetic low-rank gradient
    steps: int = 1            # optimizer steps the workload runs
    method: str = "standard"  # ns method
    hp: dict = field(default_factory=_hp)


def single_256x512() -> Workload:
    """One 256x512 fp32 matrix, three steps with a fresh rank-8 gradient each."""
    return Workload("single_256x512_fp32", [(MUON, F32, 256, 512, 0, 0)], ["w"],
                    rank=8, steps=3, hp=_hp())


def gpt2_small() -> Workload:
    """12 layers of GPT-2-small 2-D weights (fused QKV split in three 768x768
    blocks) plus the AdamW fallback on the 50257x768 embedding and 74 vectors
    of 768 (per layer ln1 w/b, ln2 w/b, attn-out bias, mlp-down bias; final LN
    w/b)."""
    t, nm = [], []
    for l in range(12):
        t += [(MUON, BF16, 2304, 768, 768, 0), (MUON, BF16, 768, 768, 0, 0),
              (MUON, BF16, 3072, 768, 0, 0), (MUON, BF16, 768, 3072, 0, 0)]
        nm += [f"h{l}.qkv", f"h{l}.attn_out", f"h{l}.mlp_up", f"h{l}.mlp_down"]
    t.append((ADAMW, BF16, 50257, 768, 0, 0))
    nm.append("wte")
    for l in range(12):
        for v in ("ln1.w", "ln1.b", "ln2.w", "ln2.b", "attn_out.b", "mlp_down.b"):
            t.append((ADAMW, BF16, 1, 768, 0, 0))
            nm.append(f"h{l}.{v}")
    t += [(ADAMW, BF16, 1, 768, 0, 0), (ADAMW, BF16, 1, 768, 0, 0)]
    nm += ["ln_f.w", "ln_f.b"]
    return Workload("gpt2_small_bf16", t, nm, rank=16)


def wide_gram(method: str = "gram") -> Workload:
    """32 wide 4096x14336 and 32 tall 14336x4096 bf16 matrices, rank 64."""
    t = [(MUON, BF16, 4096, 14336, 0, 0)] * 32 + [(MUON, BF16, 14336, 4096, 0, 0)] * 32
    nm = [f"wide{i}" for i in range(32)] + [f"tall{i}" for i in range(32)]
    return Workload(f"wide_4096x14336_{method}", t, nm, rank=64, method=method)


def llama3_8b() -> Workload:
    """32 Llama-3-8B layers {q, k, v, o, gate, up, down} in bf16, plus AdamW on
    the 128256x4096 embedding and lm_head and 65 RMSNorm vectors of 4096."""
    t, nm = [], []
    for l in range(32):
        t += [(MUON, BF16, 4096, 4096, 0, 0), (MUON, BF16, 1024, 4096, 0, 0),
              (MUON, BF16, 1024, 4096, 0, 0), (MUON, BF16, 4096, 4096, 0, 0),
              (MUON, BF16, 14336, 4096, 0, 0), (MUON, BF16, 14336, 4096, 0, 0),
              (MUON, BF16, 4096, 14336, 0, 0)]
        nm += [f"l{l}.{x}" for x in ("q", "k", "v", "o", "gate", "up", "down")]
    t += [(ADAMW, BF16, 128256, 4096, 0, 0), (ADAMW, BF16, 128256, 4096, 0, 0)]
    nm += ["embed", "lm_head"]
    for i in range(65):
        t.append((ADAMW, BF16, 1, 4096, 0, 0))
        nm.append(f"norm{i}")
    return Workload("llama3_8b_bf16", t, nm, rank=64)


def moe_grouped() -> Workload:
    """26 layers x 64 experts {gate 1408x2048, up 1408x2048, down 2048x1408},
    plus per-layer q/k/v/o 2048x2048 split into 16 head blocks of 128 rows."""
    t, nm = [], []
    for l in range(26):
        for h in ("q", "k", "v", "o"):
            t.append((MUON, BF16, 2048, 2048, 128, 0))
            nm.append(f"l{l}.{h}")
        for e in range(64):
            t += [(MUON, BF16, 1408, 2048, 0, 0), (MUON, BF16, 1408, 2048, 0, 0),
                  (MUON, BF16, 2048, 1408, 0, 0)]
            nm += [f"l{l}.e{e}.gate", f"l{l}.e{e}.up", f"l{l}.e{e}.down"]
    return Workload("moe_26x64_bf16", t, nm, rank=8)


ALL = {
    "single_256x512_fp32": single_256x512,
    "gpt2_small_bf16": gpt2_small,
    "wide_4096x14336_gram": lambda: wide_gram("gram"),
    "wide_4096x14336_standard": lambda: wide_gram("standard"),
    "llama3_8b_bf16": llama3_8b,
    "moe_26x64_bf16": moe_grouped,
}


def ns_flops(table) -> float:
    """Nominal Newton-Schulz FLOPs per iteration summed over units:
    4 m^2 n + 2 m^3 with m <= n (the metric's count)."""
    tot = 0.0
    for kind, _dt, rows, cols, split, _sd in table:
        if kind != MUON or rows == 0 or cols == 0:
            continue
        h = split if split > 0 else rows
        nb = rows // h
        m, n = min(h, cols), max(h, cols)
        tot += nb * (4.0 * m * m * n + 2.0 * m ** 3)
    return tot
