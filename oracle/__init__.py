"""CPU oracle of the MoE-layer hot path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the HIP product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
