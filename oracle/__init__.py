"""CPU oracle of the top-k routed MoE layer (test infrastructure only).

Imported by the tests, by the package smoke check and by the benchmark's
CPU-baseline leg; never by the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
