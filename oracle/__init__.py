"""CPU oracle of the DeepSeekMoE layer forward and backward (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the GPU path.  See moe_oracle.py (forward) and moe_backward.py.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__ as _fwd_all
from .moe_backward import *  # noqa: F401,F403
from .moe_backward import __all__ as _bwd_all

__all__ = list(_fwd_all) + list(_bwd_all)
