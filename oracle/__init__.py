"""fp64 CPU oracle of the mHC hyper-connection hot path.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.
"""
from .mhc_oracle import *  # noqa: F401,F403
from .mhc_oracle import __all__  # noqa: F401
