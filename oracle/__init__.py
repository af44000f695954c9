"""CPU oracle for the Q4_K SwiGLU FFN hot path -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library.
"""
from .q4k_oracle import *  # noqa: F401,F403
