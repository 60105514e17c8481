"""Plain fp64 CPU oracle of the CSA2 decode-time sparse attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.  The
product path (the HIP library and its Python binding) never calls it and shares no
code with it.
"""
from .csa2_oracle import *  # noqa: F401,F403
