"""CPU oracle of the MoE speculative verification step (test infrastructure only).

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
