"""CPU oracle of the MoE-layer forward path (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import gather_rows  # noqa: F401
