"""Plain, slow CPU oracle of the routed-expert layer (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path (``grouped_expert_amd``) never
imports it, and it never imports the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
