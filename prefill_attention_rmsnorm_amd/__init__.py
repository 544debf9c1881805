"""MI355X-native causal GQA attention path (prefill, decode, verify) and the
hidden-state RMSNorm.

The compute lives in ``libqa.so`` (hand-written HIP for gfx950, C ABI in
``include/qa.h``); ``qa`` is its ctypes binding and ``specdec`` the exact
speculative-decoding loop around ``qa.verify``.  Build with
``python -m prefill_attention_rmsnorm_amd.build``.
"""

from . import qa  # noqa: F401
from .qa import (  # noqa: F401
    Cache, Params, QaError, prefill, decode, verify, rmsnorm_hidden,
    workspace, workspace_bytes, device_error, counters, reset_counters,
)
