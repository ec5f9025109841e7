"""CPU oracle for the routed ReLU^2 MoE layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP
library.
"""
from .moe_oracle import *  # noqa: F401,F403
