"""fp64 CPU oracle for the Gated DeltaNet token mixer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may use it.
"""
from .gdn_oracle import *  # noqa: F401,F403
