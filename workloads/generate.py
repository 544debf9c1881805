"""Seeded synthetic inputs.

Every draw comes from numpy's PCG64 seeded with
``SeedSequence([workload, layer, step, tag])``; values are drawn in fp32 and
rounded once to bf16 (round to nearest even, torch's CPU conversion).  The
pages only say the workloads are fixed shapes; the distributions follow the
workload descriptions (activations ~N(0,1), projection weights ~N(0,0.02)).
"""

from __future__ import annotations

import numpy as np
import torch

TAG = {
    "q": 1, "k": 2, "v": 3, "cache_k": 4, "cache_v": 5, "emb": 6,
    "w_q": 7, "w_k": 8, "w_v": 9, "w_o": 10, "w_lm": 11, "ids": 12,
    "lens": 13, "norm_w": 14, "hidden_x": 15, "hidden_res": 16,
}


def rng(workload: int, layer: int = 0, step: int = 0, tag: str = "q"):
    """numpy Generator for one (workload, layer, step, tensor) stream."""
    ss = np.random.SeedSequence([int(workload), int(layer), int(step),
                                 TAG[tag]])
    return np.random.Generator(np.random.PCG64(ss))


def normal_bf16(shape, workload: int, layer: int = 0, step: int = 0,
                tag: str = "q", std: float = 1.0) -> torch.Tensor:
    """CPU bf16 tensor of ~N(0, std^2) draws (fp32 draw, one RNE to bf16)."""
    g = rng(workload, layer, step, tag)
    x = g.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16)


def ragged_lengths(workload: int, batch: int, choices) -> list:
    """Prompt lengths drawn i.i.d. from ``choices`` (at least two distinct).

    Draw r = 0, 1, ... until two distinct lengths appear, so the recorded
    seed always yields a genuinely ragged batch.
    """
    for r in range(1000):
        g = rng(workload, 0, r, "lens")
        lens = [int(choices[i]) for i in g.integers(0, len(choices), batch)]
        if batch < 2 or len(set(lens)) >= 2:
            return lens
    raise RuntimeError("could not draw a ragged batch")


def packed_layout(lens, start=None):
    """cu_seqlens [n+1] and per-token positions for a packed prefill.

    Sequence i's tokens sit at positions start[i] .. start[i]+lens[i]-1
    (start defaults to 0: a fresh prompt).
    """
    lens = [int(x) for x in lens]
    start = [0] * len(lens) if start is None else [int(s) for s in start]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    pos = np.concatenate([np.arange(s, s + n, dtype=np.int32)
                          for s, n in zip(start, lens)]) if lens else \
        np.zeros(0, dtype=np.int32)
    return cu, pos
