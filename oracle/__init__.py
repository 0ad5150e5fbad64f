"""fp64 CPU oracle of the MoE token-dispatch layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
