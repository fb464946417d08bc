"""CPU oracle for the sparse MoE layer forward (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
import this package; the HIP library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
