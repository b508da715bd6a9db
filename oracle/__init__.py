"""fp64 CPU oracle of the fused MoE layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
