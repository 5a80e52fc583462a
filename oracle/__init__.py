"""CPU oracle for the MC-Sparse hot path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library never does.
"""
from . import mcs_oracle  # noqa: F401
