"""Seeded synthetic workloads for the routed NVFP4 W4A4 MoE layer.

Shared input source for the oracle-side tests and the GPU path; holds no layer
arithmetic.  ``configs`` lists the five workloads, ``gen`` draws their inputs.
"""

from .configs import CONFIGS, WEIGHT_SETS, LayerConfig, WeightSet, by_name, config  # noqa: F401
from . import gen  # noqa: F401
