"""CPU oracle for query-union sparse-attention prefill over a paged FP8 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP path (no kernels, headers, helpers or tables) and
never imports ``query_union_paged_amd``; the only thing both sides share are
the seeded inputs produced by ``query_union_paged_amd.synth``.

Sources (cited by title and section; the pages are the authority on what is
computed):

* [abs]   "PageWeaver: KV-Guided Query Unions for Sparse Attention", arXiv
          2610.11201, Abstract.
* [radio] AI Radio episode "PageWeaver: KV-Guided Query Unions for Sparse
          Attention", sections "Paper summary" and "Conclusion".

Modules:

* ``fp8``        OCP e4m3fn decode and bf16 bit decode (exact, fp64).
* ``attention``  per-query sparse attention over each query's own support,
                 in fp64; the group-wise union mirror; a process-pool driver.
* ``greedy``     the bounded-window greedy grouping on Python-int bitsets.
* ``dense_union`` the direct KV-page union (disjoint page pairs, partial
                 outputs merged by log-sum-exp), in fp64.
* ``selector``   a synthetic dynamic page selector (sink + local pages + top
                 pages by block key sums), exact/fp64; our own stand-in for the
                 selection the pages take as given.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against something other than itself (library routines, closed forms, a
hand-worked example under ``tests/golden/``, an independent brute force).
The synthetic generator and the pages' published ratios are parity unpinned
(there is no recorded capture or reference output to match).
"""
