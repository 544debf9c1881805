"""Hidden-state RMSNorm in the reference's cast placement (TEST INFRASTRUCTURE ONLY).

"dryft-flash-infer" agent guide, *Where the wins are* (fused RMSNorm) and
*Numerics*: reductions may be reordered, but where the bf16 cast happens is
part of the answer.  The pages name the reference (the Qwen3 checkpoint run by
Transformers) without printing its RMSNorm; its public definition normalises
in float32, casts the normalised value to bf16, and only then multiplies by
the bf16 weight, whose product is again a bf16 tensor.  In the decoder layer
the residual stream is a bf16 tensor, so the sum entering a post-attention
norm is itself rounded to bf16 first.  That is the reading written out here,
in fp64 with every rounding explicit.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_round


def rmsnorm_hidden(x, weight=None, eps: float = 1e-6, residual=None):
    """One hidden-state norm over the last axis.

    r   = RNE_bf16(x + residual)            (r = x when residual is None)
    y   = r / sqrt(mean(r^2) + eps)          (exact fp64)
    out = RNE_bf16(weight * RNE_bf16(y))     (weight = 1 when None)

    Returns (out, r); r is the updated residual stream.  Inputs are taken as
    the values they hold (bf16 values for real tensors).
    """
    x = np.asarray(x, dtype=np.float64)
    r = x if residual is None else bf16_round(x + np.asarray(residual, dtype=np.float64))
    ms = np.mean(r * r, axis=-1, keepdims=True)
    y = bf16_round(r / np.sqrt(ms + eps))
    w = 1.0 if weight is None else np.asarray(weight, dtype=np.float64)
    return bf16_round(w * y), r
