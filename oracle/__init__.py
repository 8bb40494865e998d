"""CPU oracle for the sparse MoE layer forward pass (test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package; the HIP library never does, and this package never
imports the HIP library or its binding.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
