"""How far the greedy co-selection pairing falls from a maximum-weight matching.

TEST INFRASTRUCTURE ONLY (a CPU report over the oracle; nothing on the GPU
path imports it).  For each workload and KV head it builds the co-selection
counts of the seeded synthetic selections, pairs the pages with the greedy rule
(`affinity_pairs`) and with the exact maximum-weight matching
(`max_coselection_pairs`), and prints the (query, entry) counts per query that
each pairing leaves for the direct KV-page union ("PageWeaver: KV-Guided Query
Unions for Sparse Attention", AI Radio episode, Paper summary: disjoint page
pairs with common and exclusive query lists), and the ratio of the matched
co-selection weights.

    python -m oracle.matching_gap prefill_8k prefill_64k
"""
from __future__ import annotations

import sys
import time

from query_union_paged_amd import synth

from .dense_union import affinity_pairs, coselection, matching_weight, max_coselection_pairs


def report(name: str, workers: int = 8) -> str:
    wl = synth.WORKLOADS[name]
    sel = synth.make_selection(wl, workers=workers)
    slots = greedy = best = 0
    t_solve = 0.0
    for h in range(wl.H_kv):
        co = coselection(sel[h], wl.N)
        slots += int(((sel[h] >= 0) & (sel[h] < wl.N)).sum())
        greedy += matching_weight(co, affinity_pairs(sel[h], wl.N))
        t0 = time.time()
        best += matching_weight(co, max_coselection_pairs(sel[h], wl.N))
        t_solve += time.time() - t0
    rows = wl.T * wl.H_kv
    return (f"{name}: selected pages per query {slots / rows:.2f}; entries per query: greedy "
            f"{(slots - greedy) / rows:.3f}, maximum matching {(slots - best) / rows:.3f}; "
            f"matched weight greedy / maximum {greedy / best:.4f} (solver {t_solve:.1f} s)")


if __name__ == "__main__":
    for n in sys.argv[1:] or ["prefill_8k"]:
        print(report(n), flush=True)
