"""Float64 CPU oracle for batched paged-KV decode attention.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
statement of what the decode path computes, used to check the HIP library.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. It shares no code with the HIP path (no kernels,
headers, helpers, tables or constant generators) and imports nothing from it.

Modules, each citing the passage it follows:

* ``e4m3``      — OCP E4M3FN byte -> value, from the bit formula.
* ``e2m1``      — OCP FP4 E2M1 code -> value (two codes per byte).
* ``int4``      — two's-complement int4 code -> value (two codes per byte).
* ``storage``   — exact widening of stored K/V/q values to float64.
* ``attention`` — the definition: softmax(scale * q . K^T) . V per request and
                  query head, with K/V gathered through the page table.
* ``merge``     — partial ``(m, d, o)`` states and the online-softmax merge rule.
* ``plan``      — the work-partition rule (chunking, item order, merge index).

Every function here has a pin in ``tests/test_oracle_*.py`` that checks it
against something other than itself (brute force, closed forms, invariants,
library routines, worked examples from the pages).
"""
from . import attention, e2m1, e4m3, int4, merge, plan, storage  # noqa: F401
from .attention import decode, gather_request  # noqa: F401
