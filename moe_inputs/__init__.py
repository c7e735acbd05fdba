"""Workload definitions and seeded synthetic inputs.

Shared by both sides of every parity test (the CPU oracle and the HIP library)
and by the benchmark.  Holds no part of the layer's arithmetic.
"""
from .configs import CONFIGS, FLASH, TINY, V3, V3_FP8, V3_SKEW_EP0, MoEConfig, get  # noqa: F401
from . import generate  # noqa: F401
