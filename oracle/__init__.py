"""CPU oracle for hash-scored top-k sparse decode attention (test infrastructure).

This package is test infrastructure only.  It may be imported by ``tests/``,
by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``, and by nothing else; the GPU library never calls it and shares
no code with it.
"""
from .hst_oracle import *  # noqa: F401,F403
