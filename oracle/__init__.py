"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. It shares no code with the HIP library in
``nvfp4_weight_only_rtn_amd`` and never calls it.
"""
from .attnq_oracle import *  # noqa: F401,F403
