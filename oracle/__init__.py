"""Plain, slow fp64 CPU oracle for the OSCAR INT2 KV write and mixed-precision decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute it.  It shares no code, table or
constant generator with the HIP path (``int2_rotated_kv_write_amd``).

Every function is pinned by ``tests/test_oracle_*.py`` to facts the pages and
the mathematics fix (Hadamard closed form and lemma, bit-reversal involution,
orthogonality, hand-derived quantizer outputs, brute-force attention).
"""
from .oscar_oracle import *  # noqa: F401,F403
