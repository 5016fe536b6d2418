"""Seeded synthetic inputs for the MoE layer: workload sizes and a
counter-based generator with bit-identical host (NumPy) and device (HIP)
implementations.  Holds none of the layer's arithmetic; both the oracle
side and the HIP side of every test draw their inputs from here.
"""
from .configs import CONFIGS, ORDER, MoEConfig, small_variant  # noqa: F401
from . import rng  # noqa: F401
