"""CPU oracle of the DeepSeekMoE layer forward (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the GPU path.  See moe_oracle.py.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
