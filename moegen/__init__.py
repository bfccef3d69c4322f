"""Seeded synthetic workloads (shapes + generators) shared by the GPU path's
tests and benchmark and by the CPU oracle.  Holds no MoE-layer arithmetic."""
from .configs import *  # noqa: F401,F403
from .gen import *      # noqa: F401,F403
