"""fp64 CPU oracle for SAS gated block-sparse attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may use it.
"""
from .sas_oracle import *  # noqa: F401,F403
from . import sas_oracle  # noqa: F401
