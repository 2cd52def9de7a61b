"""Workload shapes for the single-GPU MoE-layer forward path.

Each shape follows the problem statement used throughout the pages: T tokens of
hidden size d, E experts, top-k routing, expert intermediate size f, plus the
routing options (group-limited pre-selection, partial top-P pre-selection, gate
renormalisation), the number of expert-parallel ranks whose send layout is
emitted, the compute dtype and the kind of per-expert logit bias used to create
load imbalance.

This module holds shapes only; no arithmetic of the method lives here.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int          # tokens
    d: int          # hidden size
    E: int          # experts
    k: int          # experts chosen per token
    f: int          # expert intermediate size (SwiGLU)
    n_group: int = 1      # expert groups for group-limited selection (1 = off)
    topk_group: int = 1   # groups kept per token
    presel: int = 0       # 0 = off; else softmax over the best `presel` scores
    renorm: int = 1       # 1 = gates renormalised over the k chosen experts
    ep_ranks: int = 1     # ranks of the emitted expert-parallel send layout
    dtype: str = "bf16"   # "bf16" or "f32" (activations and weights)
    bias: str = "none"    # "none" | "normal" (b_e ~ N(0,1)) | "zipf" (b_e = -1.1 ln(e+1))
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def A(self) -> int:
        """Rows of the expert-contiguous buffers: one per (token, choice)."""
        return self.T * self.k

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)


# The five workloads, in order (the first is the small fp32 case).
TINY_F32 = MoEShape("tiny-f32-T256-d64-E8-top2-f128", T=256, d=64, E=8, k=2, f=128,
                    dtype="f32", ep_ranks=1)
E8_D4096 = MoEShape("T1024-d4096-E8-top2-f11008", T=1024, d=4096, E=8, k=2, f=11008,
                    ep_ranks=2)
E64_PRESEL8 = MoEShape("T4096-d2048-E64-presel8-top2-f1408-biasN01", T=4096, d=2048, E=64,
                       k=2, f=1408, presel=8, renorm=0, ep_ranks=8, bias="normal")
E16_ZIPF = MoEShape("T16384-d5120-E16-top2-f1536-zipf", T=16384, d=5120, E=16, k=2, f=1536,
                    ep_ranks=4, bias="zipf")
E256_GROUPED = MoEShape("T8192-d7168-E256-g8x4-top8-f2048", T=8192, d=7168, E=256, k=8,
                        f=2048, n_group=8, topk_group=4, ep_ranks=64)

CONFIGS = [TINY_F32, E8_D4096, E64_PRESEL8, E16_ZIPF, E256_GROUPED]
BY_NAME = {c.name: c for c in CONFIGS}

# Reduced shapes with the same routing structure, small enough for the CPU
# oracle to finish in seconds while still spanning several GEMM tiles and a
# ragged tail of rows per expert.
SMALL = {
    "tiny": TINY_F32,
    "e8": E8_D4096.replace(name="small-e8", T=300, d=256, f=448),
    "e64": E64_PRESEL8.replace(name="small-e64-presel8", T=520, d=256, f=192),
    "e16": E16_ZIPF.replace(name="small-e16-zipf", T=700, d=320, f=256),
    "e256": E256_GROUPED.replace(name="small-e256-grouped", T=400, d=512, f=192),
}
