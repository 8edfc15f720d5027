"""fp64 CPU oracle for TPLA decode attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package.  It shares no code with the HIP library.
"""
from .tpla_oracle import *  # noqa: F401,F403
from .tpla_oracle import __all__  # noqa: F401
