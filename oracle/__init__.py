"""CPU oracle of the MoE layer -- test infrastructure, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library under ``mixture_experts_layer_permute_amd/`` and imports nothing
from it.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
from ._cbuild import build as build_c  # noqa: F401
