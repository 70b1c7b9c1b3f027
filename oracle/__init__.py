"""CPU oracle of the MoE decode layer (test infrastructure only).

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import this package.  The product path never calls it.
"""
from .moe_oracle import *  # noqa: F401,F403
