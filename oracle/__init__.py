"""CPU oracle for byte-level BPE (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does.
"""
from .oracle import *  # noqa: F401,F403
