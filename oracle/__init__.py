"""CPU oracle of the routed sparse-MoE layer: test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline legs
(``cpu_baseline``, ``cpu_baseline_cxx``) of ``bench.py``; never by the product
library.  ``moe_oracle`` is the numpy oracle, ``oracle_c`` binds the C++ one.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
