"""CPU oracle of the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Imported only by the tests, the smoke check and the benchmark's CPU-baseline leg;
the product path never imports, links or runs anything here.
"""
from . import moe_oracle  # noqa: F401
from .moe_oracle import *  # noqa: F401,F403
