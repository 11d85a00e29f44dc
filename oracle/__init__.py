"""CPU oracle for the Kitty mixed-precision 2-bit KV cache hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything under
``oracle/``.  The product path (the HIP library and its Python binding) never
imports it, and it shares no code, table or constant generator with it.

Parity status: every function in ``kitty_oracle`` is pinned by a CPU test in
``tests/test_oracle.py`` against something other than itself (the pages'
printed avg-bits table, closed forms, exact-rational brute force, textbook
min/max quantization as a special case, fp64 brute-force attention and torch
SDPA).  No function is "parity unpinned"; the attention tolerance (2e-3 max
abs) is the one fixed for this build, the pages give no error bound.
"""
from .kitty_oracle import *  # noqa: F401,F403
