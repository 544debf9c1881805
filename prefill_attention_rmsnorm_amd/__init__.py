"""MI355X-native causal GQA attention path (prefill, decode, verify).

The compute lives in ``libqa.so`` (hand-written HIP for gfx950, C ABI in
``include/qa.h``); ``qa`` is its ctypes binding.  Build with
``python -m prefill_attention_rmsnorm_amd.build``.
"""

from . import qa  # noqa: F401
from .qa import (  # noqa: F401
    Cache, Params, QaError, prefill, decode, verify, workspace,
    workspace_bytes, device_error, counters, reset_counters,
)
