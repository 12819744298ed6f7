"""CPU oracle (fp64) for frame-windowed sparse attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library itself.
"""
from .fsa_oracle import *  # noqa: F401,F403
from .fsa_oracle import __all__  # noqa: F401
