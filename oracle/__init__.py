"""fp64 CPU oracle for the causal GQA attention path (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, obviously-correct definition that the HIP
kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product library
never does, and the oracle imports nothing from the product.

Sources (web pages, cited by title and section):

* "dryft-flash-infer" agent guide -- *Invariants* (greedy choice within 2.0
  logits of the argmax), *Where the wins are* (preallocated strided KV cache;
  fused RMSNorm and rotary embedding; exact speculative verification),
  *Numerics* (reorderings and fp32 accumulation are within budget, moving the
  bf16 cast is not).
* "htn.dryft.ai/docs" -- *What to submit* (a batch of token sequences stepped
  one token per sequence per step; the Qwen3-4B-Instruct-2507 bf16 checkpoint
  on one H100) and *Scoring and correctness*.

Functions and what pins each of them (tests under ``tests/test_oracle_*``):

=====================  ====================================================
``bf16_round``          torch CPU ``.to(bfloat16)`` on ties/subnormals/inf/NaN
``rmsnorm``             closed forms (RMS of output, constant vector, a
                        hand-computed 2-vector with and without weight)
``rope``                identity at p=0, per-pair norm, composition,
                        relative-position identity, 50-digit complex twin,
                        hand values cos(1)/sin(1) at chosen (i, p)
``attend_rows``         single key, uniform V, q=0, two-key sigmoid, shift
                        and permutation invariance, torch fp64 SDPA with an
                        explicit bottom-right mask, 50-digit brute force
``prefill/decode/verify``  causality, decode == prefill row, verify ==
                        sequential decodes, packed == separate, GQA == MHA
``rmsnorm_hidden``      hand values incl. a tie and the cast-placement case,
                        constant vectors, torch CPU bf16 add and the
                        float32 reference arithmetic
``o_proj``,             hand values (a tie, the cast before the residual add),
``attn_epilogue``       exact rational sums on small shapes, identity and
                        zero weights, torch CPU bf16 linear layer
``lm_logits``           50-digit brute force on tiny shapes
``margin_ok``           rule cases (tie, exactly 2.0 below, just over)
=====================  ====================================================

Readings of the pages that the pins cannot decide (the pages give no worked
numbers for any of these): the rotate-half RoPE pairing, the frequency rule
theta^(-2i/d) and the single bf16 rounding of k at the cache write.  Each is
pinned to its own mathematical definition above; whether it is the pages'
convention is *parity unpinned* by the pages.
"""

from .attention import (  # noqa: F401
    bf16_round,
    bf16_bits,
    bits_to_f64,
    rmsnorm,
    rope_inv_freq,
    rope,
    attend_rows,
    Cache,
    write_kv,
    attend_tokens,
    prefill,
    decode,
    verify,
    lm_logits,
    margin_ok,
    argmax_lowest,
)
from .rmsnorm_hidden import rmsnorm_hidden  # noqa: F401
from .epilogue import o_proj, attn_epilogue  # noqa: F401
