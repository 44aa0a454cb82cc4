"""CPU oracle of the Stable LatentMoE layer (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package.  It shares no code with the HIP path.
"""
from . import moe_oracle  # noqa: F401
