"""Seeded synthetic inputs and the literal workload configurations.

Serves both the HIP path (tests, bench) and the fp64 oracle; holds none of
the method's arithmetic.
"""

from .configs import CONFIGS, LayerConfig, scaled
from .gen import generate, sink_positions, head_factors

__all__ = ["CONFIGS", "LayerConfig", "scaled", "generate", "sink_positions",
           "head_factors"]
