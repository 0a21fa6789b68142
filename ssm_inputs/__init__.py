"""Seeded synthetic workloads shared by tests, the oracle side and the benchmark.

Holds no part of the scan's arithmetic (see ``generate.py``).
"""
from . import configs, generate  # noqa: F401
from .configs import (TINY_FP32, MAMBA130M_LAYER, MAMBA2P8B_LAYER,  # noqa: F401
                      LONG_CONTEXT_1M, DECODE_256x8192, PACKED_2P8B_LAYER, FUSED_2P8B_LAYER,
                      PackedConfig, ScanConfig, StepConfig)
