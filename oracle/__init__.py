"""CPU oracle for the TurboQuant KV-cache hot path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  It shares no code with the HIP library and imports nothing
from it.
"""
from .tq_oracle import *  # noqa: F401,F403
from . import tq_oracle  # noqa: F401
