"""fp64 CPU oracle for causal kernelized linear attention.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
"""

from .linear_attention import *  # noqa: F401,F403
from .linear_attention import __all__  # noqa: F401
