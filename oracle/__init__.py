"""fp64 CPU oracle for exact attention: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the HIP product path never does.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
