"""Workload shapes for SparK prefill pruning and decode attention.

Each workload is one attention layer shaped like LLaMA-3.1-8B (32 query heads,
8 KV heads, head dim 128) unless stated. The SparK pages (the Chinese
walkthrough of arXiv 2508.15212, sections 3.2-3.3 and 4.3) give the method and
the context lengths (up to 128K in Fig. 4b); the numbers here fix the batch,
sequence length, pruning ratio and observation window of each synthetic run.
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int          # seed component: keeps the random streams of workloads apart
    B: int
    S: int
    n_q: int
    n_kv: int
    D: int
    window: int
    lam: float           # fraction of key channels pruned
    steps: int           # decode steps after one prefill prune
    layers: int = 1
    keep: Optional[int] = None   # tokens kept per KV head by window-score eviction (stacked case)

    @property
    def G(self) -> int:
        return self.n_q // self.n_kv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny single layer: the size the CPU oracle finishes in seconds
    "tiny_s1k": Workload("tiny_s1k", 0, 1, 1024, 32, 8, 128, 32, 0.5, 1),
    # LLaMA-3.1-8B-shaped single layer at 32K context
    "llama8b_s32k_l05": Workload("llama8b_s32k_l05", 1, 1, 32768, 32, 8, 128, 32, 0.5, 64),
    "llama8b_s32k_l08": Workload("llama8b_s32k_l08", 1, 1, 32768, 32, 8, 128, 32, 0.8, 64),
    # the ~100K-context case
    "llama8b_s128k_l08": Workload("llama8b_s128k_l08", 2, 1, 131072, 32, 8, 128, 32, 0.8, 64),
    # window-score eviction to 4096 tokens per KV head, then channel pruning
    "snapkv_b8_s32k_keep4k_l07": Workload("snapkv_b8_s32k_keep4k_l07", 3, 8, 32768, 32, 8, 128, 32, 0.7, 64,
                                          keep=4096),
    # full 32-layer KV stack
    "llama8b_32L_b4_s64k_l08": Workload("llama8b_32L_b4_s64k_l08", 4, 4, 65536, 32, 8, 128, 32, 0.8, 64,
                                        layers=32),
}
