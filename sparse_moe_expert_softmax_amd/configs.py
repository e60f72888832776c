"""Workload shapes for the MoE-layer forward (router, expert FFNs, combine).

Shapes follow the FreeToken pages where they give one (the explainer page,
"why now" section: 256 experts, 6 active, 43 MoE layers for the 284B/13B
model; "how" section: 8,192-token prefill chunks) and otherwise the plain
reading of the workload description (hidden, intermediate, top-k, formats).
This module holds sizes only: no arithmetic of the method lives here.
"""
from dataclasses import dataclass, field
from typing import Tuple

# weight / activation element formats (values match ft_dtype in ft_moe.h)
F32, BF16, MXFP4, NVFP4 = 0, 1, 2, 3
DTYPE_NAMES = {F32: "f32", BF16: "bf16", MXFP4: "mxfp4", NVFP4: "nvfp4"}


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cid: int                 # stable small integer, part of every seed
    hidden: int              # H
    inter: int               # I (per-expert SwiGLU width)
    n_experts: int           # E
    top_k: int               # k
    act_dtype: int           # x
    router_dtype: int        # W_r
    w_dtype: int             # expert weights
    n_layers: int
    batches: Tuple[int, ...] = (1,)
    renormalize: bool = True
    weight_std: float = 0.02
    pool_fraction: float = 1.0   # fraction of all (layer, expert) keys the slot pool holds
    trace_steps: int = 0
    zipf_s: float = 0.0
    n_masks: int = 0
    note: str = ""

    @property
    def n_slots(self) -> int:
        return int(self.pool_fraction * self.n_experts * self.n_layers)


C1 = MoEConfig("tiny_f32", 1, hidden=256, inter=512, n_experts=8, top_k=2,
               act_dtype=F32, router_dtype=F32, w_dtype=F32, n_layers=1,
               batches=(16,), note="tiny fp32 layer, 16 tokens")
C2 = MoEConfig("decode_bf16_h2048_e128", 2, hidden=2048, inter=768, n_experts=128, top_k=8,
               act_dtype=BF16, router_dtype=BF16, w_dtype=BF16, n_layers=40,
               batches=(1, 2, 4), note="35B-A3B-like decode, all experts resident")
C3 = MoEConfig("decode_mxfp4_h4096_e256_lru", 3, hidden=4096, inter=2048, n_experts=256, top_k=6,
               act_dtype=BF16, router_dtype=BF16, w_dtype=MXFP4, n_layers=43,
               batches=(1, 2, 3, 4), pool_fraction=0.25, trace_steps=2048, zipf_s=1.1,
               note="284B/13B-like decode through a global LRU slot pool")
C4 = MoEConfig("prefill_mxfp4_h4096_e256", 4, hidden=4096, inter=2048, n_experts=256, top_k=6,
               act_dtype=BF16, router_dtype=BF16, w_dtype=MXFP4, n_layers=43,
               batches=(8192, 16384), note="prefill chunk of 8,192 tokens")
C5 = MoEConfig("decode_nvfp4_h6144_e256", 5, hidden=6144, inter=2048, n_experts=256, top_k=8,
               act_dtype=BF16, router_dtype=BF16, w_dtype=NVFP4, n_layers=8,
               batches=(4,), n_masks=16, note="753B/40B-like decode with 50/50 partition masks")

C6 = MoEConfig("prefill_bf16_h2048_e128", 6, hidden=2048, inter=768, n_experts=128, top_k=8,
               act_dtype=BF16, router_dtype=BF16, w_dtype=BF16, n_layers=40,
               batches=(8192,), note="prefill chunk of 8,192 tokens through the 35B-like bf16 layer")

C7 = MoEConfig("prefill_nvfp4_h6144_e256", 7, hidden=6144, inter=2048, n_experts=256, top_k=8,
               act_dtype=BF16, router_dtype=BF16, w_dtype=NVFP4, n_layers=8,
               batches=(8192,), note="prefill chunk of 8,192 tokens through the 753B-like NVFP4 layer")

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5, C6, C7)}
BY_ID = {c.cid: c for c in (C1, C2, C3, C4, C5, C6, C7)}
