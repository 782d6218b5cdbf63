"""fp64 CPU oracle for exact attention: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the HIP product path never does.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__ as _attention_all
from .dropout import *  # noqa: F401,F403
from .dropout import __all__ as _dropout_all

__all__ = list(_attention_all) + list(_dropout_all)
