"""Bounded-window greedy grouping of queries by selected-page affinity.

From the pages: a bounded GPU search produces query IDs and nothing else
("PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract); within a
bounded window the members of a query-owned group are collected greedily,
each time taking a query whose selected set adds few new pages to the group,
and the group size g = 8 is fixed independently of the window W (AI Radio
episode on the paper, section "Paper summary").

Readings taken where the pages leave a step open:

* windows are disjoint aligned blocks of W consecutive query IDs per KV head
  (the last one may be shorter);
* the lowest unassigned ID of the window owns (seeds) the next group;
* the cost of a candidate c is the number of its pages not yet in the group's
  union U, |S_c \\ U|, counted in pages; ties go to the lowest query ID;
* a group closes at g members or when the window runs out of candidates;
* IDs are emitted window by window, group by group, members in insertion
  order (seed first);
* each KV head is grouped independently.

Supports are Python ints used as bitsets (bit u set iff page u is selected);
the step is written out directly with ``int.bit_count``.
"""
from __future__ import annotations

import os
from typing import List, Optional

import numpy as np


def support_bits(row: np.ndarray, N: int) -> int:
    b = 0
    for u in row.tolist():
        if 0 <= u < N:
            b |= 1 << u
    return b


def greedy_window(bits: List[int], g: int) -> List[int]:
    """Greedy grouping of one window; returns local indices in emission order."""
    remaining = list(range(len(bits)))        # kept ascending
    order: List[int] = []
    while remaining:
        seed = remaining.pop(0)               # lowest unassigned ID
        group = [seed]
        union = bits[seed]
        while len(group) < g and remaining:
            best = None
            best_cost = None
            for c in remaining:               # ascending, so strict < keeps lowest ID on ties
                cost = (bits[c] & ~union).bit_count()
                if best_cost is None or cost < best_cost:
                    best, best_cost = c, cost
            remaining.remove(best)
            group.append(best)
            union |= bits[best]
        order.extend(group)
    return order


def group_head(sel_h: np.ndarray, N: int, W: int, g: int) -> np.ndarray:
    """int32 [T] query IDs for one KV head."""
    T = sel_h.shape[0]
    out = np.empty(T, dtype=np.int32)
    for w0 in range(0, T, W):
        w1 = min(T, w0 + W)
        bits = [support_bits(sel_h[t], N) for t in range(w0, w1)]
        out[w0:w1] = np.array(greedy_window(bits, g), dtype=np.int32) + w0
    return out


def _group_windows(args):
    sel_h, N, W, g, w_list = args
    res = []
    for w0 in w_list:
        w1 = min(sel_h.shape[0], w0 + W)
        bits = [support_bits(sel_h[t], N) for t in range(w0, w1)]
        res.append((w0, np.array(greedy_window(bits, g), dtype=np.int32) + w0))
    return res


def group_ids(sel: np.ndarray, N: int, W: int, g: int,
              workers: Optional[int] = None, windows: Optional[dict] = None) -> np.ndarray:
    """int32 [H_kv][T] query IDs.

    ``windows`` (optional) maps head -> list of window starts to compute; the
    other entries are left as -1.  ``workers > 1`` uses a process pool."""
    H, T, _ = sel.shape
    out = np.full((H, T), -1, dtype=np.int32)
    jobs = []
    for h in range(H):
        starts = list(range(0, T, W)) if windows is None else list(windows.get(h, []))
        n = max(1, len(starts) // 8)
        for i in range(0, len(starts), n):
            jobs.append((h, (sel[h], N, W, g, starts[i:i + n])))
    workers = workers if workers is not None else 1
    if workers > 1 and len(jobs) > 1:
        import multiprocessing as mp
        pool = mp.get_context("fork").Pool(workers)
        try:
            results = pool.map(_group_windows, [j for _, j in jobs])
        finally:                     # let workers exit on their own (no SIGTERM)
            pool.close()
            pool.join()
    else:
        results = [_group_windows(j) for _, j in jobs]
    for (h, _), res in zip(jobs, results):
        for w0, ids in res:
            out[h, w0:w0 + ids.size] = ids
    return out


def default_workers() -> int:
    return len(os.sched_getaffinity(0))
