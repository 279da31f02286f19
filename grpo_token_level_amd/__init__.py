"""Token-level GRPO policy-loss hot path for AMD MI355X (gfx950).

The compute lives in ``libgrpo.so`` (host C++ plans / advantage / accumulator
and hand-written HIP kernels), declared in ``include/grpo.h``.  This package
is its Python binding (``ops``) plus the build step (``build``).
"""

from . import ops  # noqa: F401
from .ops import GrpoError  # noqa: F401
