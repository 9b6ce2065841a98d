"""Seeded synthetic workloads for the selective scan (input generation only).

Shared by the CPU oracle's tests and by the GPU path's tests and benchmark; it
holds no step of the scan's arithmetic.
"""
from .configs import CONFIGS, BY_NAME, ScanConfig, TINY, M130, B28, LONG, DECODE, tolerance  # noqa: F401
from . import inputs, philox  # noqa: F401
