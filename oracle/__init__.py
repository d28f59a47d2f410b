"""fp64 CPU oracle of the routed MoE FFN layer -- test infrastructure only.

Imported by the test suite, the smoke check and the benchmark's CPU-baseline
leg; never by the library or its binding.  See moe_oracle for the definition
and the page passages each step follows.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import Route  # noqa: F401
