"""CPU oracle for the MoE token-dispatch layer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
