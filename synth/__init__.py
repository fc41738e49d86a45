"""Seeded synthetic inputs shaped like the pages' decode workloads.

This package holds no arithmetic of the method: it draws random tensors, block
tables and sequence lengths and nothing else.  It is the only code shared by the
HIP path's tests/benchmark and the CPU oracle.
"""

from .configs import CONFIGS, LayerKind, Workload, workload  # noqa: F401
from . import gen  # noqa: F401
