"""CPU oracle for the HLQ/HOT linear-layer backward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it.
"""
from .hlq_oracle import *  # noqa: F401,F403
