"""CPU oracle for the MoE dispatch -> grouped gated-SiLU expert MLP -> combine path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (``combine_top_expert_amd``)
imports, calls or links anything in this package; only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, tables or helpers with the HIP path.

Plain, slow, obviously correct: numpy, fp64 dot products, Python loops where
the pages describe a sequential procedure.  Each function cites the page
passage it follows; see ``formats`` (number formats), ``moe`` (the path),
``router`` (the router top-k step in front of it) and ``backward`` (the
gradients of the path, in the reverse order).

Every function here is pinned by ``tests/test_oracle_*.py`` against facts the
pages print, closed forms, invariants, library routines or brute force.
"""
from . import backward, formats, moe, router  # noqa: F401
