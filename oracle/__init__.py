"""CPU oracle for the AWQ W4A16 hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product (the HIP library and its Python
binding) imports, links or runs anything in this package. Only the tests, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py``
may use it.
"""

from .awq_oracle import *  # noqa: F401,F403
