"""Scalar fp64 CPU oracle for the streaming-MoE decode step (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
use this package. It wraps ``oracle.cpp`` (plain loops, double precision)
through ctypes and shares nothing with the HIP library.
"""

from .oracle import *  # noqa: F401,F403
from .oracle import build, load  # noqa: F401
