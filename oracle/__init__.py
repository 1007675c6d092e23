"""CPU oracle of the MoE layer's hot path -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It imports nothing from the HIP library's package.
"""
from . import moe_oracle  # noqa: F401
from .moe_oracle import *  # noqa: F401,F403
