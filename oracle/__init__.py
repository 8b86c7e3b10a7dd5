"""CPU oracle of the fused MoE forward — test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library.
"""
from . import moe_oracle  # noqa: F401
