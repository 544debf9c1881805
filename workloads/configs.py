"""The five workloads of the attention path, as data.

Shapes follow the pages' public workload ranges ("dryft-flash-infer" agent
guide, *What is measured* and *Where the wins are*: batch 1 and 4, prompts of
512 to 2048 tokens, outputs of 32 to 128 tokens) and the Qwen3-4B head layout
named in "htn.dryft.ai/docs", *What to submit* (32 query heads, 8 KV heads,
head_dim 128, hidden 2560).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    prompt_lens: tuple  # per sequence; empty for ragged (drawn by seed)
    decode_steps: int
    capacity: int
    verify_block: int = 0
    verify_start: int = 0
    vocab: int = 0
    theta: float = 1.0e6
    eps: float = 1.0e-6
    ragged_choices: tuple = field(default=())

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = (
    # Tiny closed loop: 64-token prompt, 8 greedy steps through a random LM head.
    Workload("tiny", 0, batch=1, n_layers=1, n_q_heads=4, n_kv_heads=1,
             head_dim=128, hidden=2560, prompt_lens=(64,), decode_steps=8,
             capacity=72, vocab=151936),
    # One Qwen3-4B attention layer, batch 1, prompt 512, 32 decode steps.
    Workload("qwen3_4b_b1_s512", 1, batch=1, n_layers=1, n_q_heads=32,
             n_kv_heads=8, head_dim=128, hidden=2560, prompt_lens=(512,),
             decode_steps=32, capacity=544),
    # Batch 4, prompts of 2048, 128 decode steps over all 36 layers' caches.
    Workload("qwen3_4b_b4_s2048_36l", 2, batch=4, n_layers=36, n_q_heads=32,
             n_kv_heads=8, head_dim=128, hidden=2560,
             prompt_lens=(2048, 2048, 2048, 2048), decode_steps=128,
             capacity=2176),
    # Ragged batch 4: prompt lengths drawn from {512, 1024, 1536, 2048}.
    Workload("qwen3_4b_ragged_b4", 3, batch=4, n_layers=1, n_q_heads=32,
             n_kv_heads=8, head_dim=128, hidden=2560, prompt_lens=(),
             decode_steps=64, capacity=2112,
             ragged_choices=(512, 1024, 1536, 2048)),
    # Exact verification of a 16-token draft block after a 2048-slot cache.
    Workload("qwen3_4b_verify_b4_k16", 4, batch=4, n_layers=1, n_q_heads=32,
             n_kv_heads=8, head_dim=128, hidden=2560, prompt_lens=(),
             decode_steps=0, capacity=2064, verify_block=16,
             verify_start=2048, vocab=151936),
)


def get(key) -> Workload:
    """Workload by index or name."""
    for w in WORKLOADS:
        if key == w.index or key == w.name:
            return w
    raise KeyError(key)
