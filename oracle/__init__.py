"""CPU oracle (test infrastructure only; see oracle/attention.py).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The GPU library never does, and it has no fallback to it.
"""
from .attention import backward, decode, forward, lengths, preprocess, probabilities  # noqa: F401
from . import rope  # noqa: F401
