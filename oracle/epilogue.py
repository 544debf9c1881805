"""Attention epilogue in the reference's cast placement (TEST INFRASTRUCTURE ONLY).

"dryft-flash-infer" agent guide, *Where the wins are* ("Fused kernels": RMSNorm,
rotary embedding and the attention epilogue) and *Numerics* (reductions may be
reordered and accumulated in fp32, but where the bf16 cast happens is part of
the answer).  The pages name the reference (the Qwen3 checkpoint under
Transformers) without printing its decoder layer.  Its public definition after
attention: the output projection, a bf16 linear layer whose weight is
[hidden, n_q_heads * head_dim] (one row per output feature) and whose sums are
rounded to bf16 once; the residual add in the bf16 residual stream; then the
post-attention RMSNorm (``rmsnorm_hidden``).  Written out here in fp64 with
every rounding explicit.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_round
from .rmsnorm_hidden import rmsnorm_hidden


def o_proj(o_flat, w_o) -> np.ndarray:
    """h = RNE_bf16(o_flat @ w_o^T).

    o_flat [T, in_dim] (the attention output, heads concatenated), w_o
    [hidden, in_dim].  The products of bf16 values are exact in fp64 and the
    sums carry fp64 rounding only; the single rounding to bf16 follows.
    """
    o = np.asarray(o_flat, dtype=np.float64)
    w = np.asarray(w_o, dtype=np.float64)
    return bf16_round(o @ w.T)


def attn_epilogue(o_flat, w_o, residual, weight=None, eps: float = 1e-6):
    """The epilogue of one attention block.

    h   = RNE_bf16(o_flat @ w_o^T)                       (output projection)
    r   = RNE_bf16(residual + h)                         (the new residual stream)
    out = RNE_bf16(weight * RNE_bf16(r / sqrt(mean(r^2) + eps)))

    Returns (out, r, h).
    """
    h = o_proj(o_flat, w_o)
    out, r = rmsnorm_hidden(h, weight, eps, residual)
    return out, r, h
