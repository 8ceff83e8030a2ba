"""CPU oracle of the CSA2 hot path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and it imports nothing from the library.
"""
from . import formats, csa2  # noqa: F401
