"""Workload shapes and seeded synthetic inputs shared by tests, smoke and bench.

This package holds no attention arithmetic: only shapes (``configs``) and
random draws (``generate``).  Both the HIP path and the oracle consume what it
produces; neither is imported here.
"""

from .configs import WORKLOADS, Workload, get  # noqa: F401
from .generate import (  # noqa: F401
    TAG,
    rng,
    normal_bf16,
    ragged_lengths,
    packed_layout,
)
