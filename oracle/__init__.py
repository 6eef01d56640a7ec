"""fp64 CPU oracle of gist-token sparse attention.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
bench's CPU-baseline leg.  Nothing in the library path may import it.
"""
from .gsa_oracle import *  # noqa: F401,F403
from .gsa_oracle import Layout, TypeMap, type_map, select, attend, block_table  # noqa: F401
