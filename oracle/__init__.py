"""fp64 CPU oracle of the fused Dynamic Tanh layer and its tolerance checks.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg. The HIP library never uses it.
"""
from . import compare, dyt_oracle  # noqa: F401
from .dyt_oracle import backward, forward  # noqa: F401
