"""MI355X (gfx950) attention-state library for sequence-parallel DiT inference.

Partition-wise exact attention emitting states AS(i) = (OUT(i), LSE(i)), their
log-sum-exp composition, and LSE-derived partition weights, implemented as HIP
kernels behind the C ABI of include/as_attn.h. This package holds the ctypes
binding (``_native``), a thin composition of library calls for the
selective-reuse step (``reuse``), the seeded synthetic workloads (``inputs``)
and the in-tree build (``build``).
"""
from ._native import (  # noqa: F401
    ASError,
    contribution_workspace_size,
    merge,
    partition_attn,
    partition_contribution,
)
