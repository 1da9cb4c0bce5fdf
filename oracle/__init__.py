"""CPU oracle for the MLA latent-cache path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it; the two meet only in the seeded input arrays built by
``mla_latent_kv_22_amd.inputs``.
"""
from .mla_oracle import *  # noqa: F401,F403
