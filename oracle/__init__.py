"""Plain, slow CPU oracle for block-sparse paged attention (fp64 numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, header, table or helper with the HIP
library under ``block_sparse_paged_bsr_amd/``; the two meet only through the seeded
inputs of ``workloads.py`` (repository root), which hold no attention or
planning arithmetic.

Modules
-------
``attention``  exact attention over a paged/BSR KV cache, the attention state (O, LSE)
               and the merge operator; every function names the passage it follows.
``plan``       the load-balanced split-KV partition (longest-processing-time greedy)
               written step by step in the pages' order.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against
values the pages print, closed forms, a library routine in special cases, or
invariants.  The slot *numbering* inside the reduction map is not fixed by any page
("parity unpinned" for that numbering convention only); it is checked against the
HIP library's planner, and its structure (which partials feed which output, in which
order) is pinned.
"""
