"""CPU fp64 oracle for the sigmoid-routed Q4 MoE expert layer (test infrastructure).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this package.  The GPU library never
imports, links or calls anything here, and nothing here imports the GPU
library: the two share no code.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
