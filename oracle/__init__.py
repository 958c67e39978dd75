"""fp64 CPU oracle for the KDA state recurrence (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package.  The HIP library never does.
"""
from .kda_oracle import *  # noqa: F401,F403
