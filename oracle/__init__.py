"""CPU fp64 oracle of the decode-time fine-grained MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and imports nothing from it.
"""
from .moe_ref import *  # noqa: F401,F403
