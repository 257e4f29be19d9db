"""Float64 CPU oracle for DMS attention.

TEST INFRASTRUCTURE ONLY: importable from ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never from the product package.
"""

from . import bruteforce, dms_oracle, soft_mask  # noqa: F401
