"""CPU oracle for the Sparse-BitLinear hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and it shares no code
with that path: the two meet only in ``workloads.py``, which draws inputs and
holds none of the method's arithmetic.

See ``oracle/sbn_oracle.py`` for the definitions and their citations.
"""
from .sbn_oracle import *  # noqa: F401,F403
