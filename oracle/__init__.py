"""Plain fp64 CPU oracle for partition-wise attention states.

TEST INFRASTRUCTURE, not product code. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package. It shares no code with the HIP path
(``sequence_dit_amd``) and imports nothing from it: it takes numpy/torch CPU
arrays and returns float64 numpy arrays.

Parity pinning: every function here is pinned by ``tests/test_oracle.py``
against library routines, closed forms, invariants and a hand-worked example
(``tests/golden/``). No function is "parity unpinned".
"""
from .states import (  # noqa: F401
    compose_groups,
    contribution,
    full_attention,
    merge,
    merge_pair,
    mse,
    nearest_partitions,
    partition_states,
    selective_reuse,
)
from . import planner  # noqa: F401  (anchor-guided planner statistics)
from . import fp8  # noqa: F401  (E4M3 codes -> values for the fp8-input path)
