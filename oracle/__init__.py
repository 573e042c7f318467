"""CPU oracle (test infrastructure only; never imported by the product path).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.
"""
from .dsa_oracle import *  # noqa: F401,F403
from .dsa_oracle import __all__  # noqa: F401
