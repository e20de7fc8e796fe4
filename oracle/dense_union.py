"""Direct KV-page union (the pages' complementary design study), in fp64.

The pages contrast query groups with a direct KV-page union that studies
non-local reuse against its reduction cost ("PageWeaver: KV-Guided Query
Unions for Sparse Attention", Abstract); it works on disjoint page pairs and
uses the full membership of each page to form common and exclusive query lists
(AI Radio episode on the paper, section "Paper summary").  Unlike the query
union it produces one partial output per (query, page pair), so the per-query
results have to be merged afterwards.

Readings taken: pages are paired by ID as (2k, 2k+1); the full membership of a
pair is every query of that KV head that selected either page; the common list
holds the queries that selected both, the exclusive lists those that selected
exactly one of them; each (query, Q head, pair) partial is (m, l, acc) over the
query's own visible keys in the pair; partials are merged by log-sum-exp.  The
merged result is the same O as ``oracle.attention`` (only the order of the
floating-point work differs).
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np

from .attention import Problem


def pair_lists(pb: Problem, h: int) -> Dict[int, Dict[str, List[int]]]:
    """pair k -> {'common': [...], 'only_even': [...], 'only_odd': [...]}, sorted query IDs."""
    lists: Dict[int, Dict[str, List[int]]] = {}
    for t in range(pb.T):
        sup = set(pb.support(h, t).tolist())
        for k in sorted({u // 2 for u in sup}):
            has_e, has_o = (2 * k) in sup, (2 * k + 1) in sup
            kind = "common" if (has_e and has_o) else ("only_even" if has_e else "only_odd")
            lists.setdefault(k, {"common": [], "only_even": [], "only_odd": []})[kind].append(t)
    return lists


def dense_union(pb: Problem) -> np.ndarray:
    """O as fp64 [T][H_q][D] via per-pair partials and a log-sum-exp merge."""
    G, D, P = pb.G, pb.D, pb.P
    out = np.zeros((pb.T, pb.H_q, D))
    for h in range(pb.H_kv):
        kh, vh = pb.k_hat(h), pb.v_hat(h)
        partials: Dict[int, list] = {}
        for k, kinds in sorted(pair_lists(pb, h).items()):
            for kind, members in kinds.items():
                pages = {"common": [2 * k, 2 * k + 1], "only_even": [2 * k],
                         "only_odd": [2 * k + 1]}[kind]
                pos = (np.array(pages)[:, None] * P + np.arange(P)[None, :]).ravel()
                kk = kh[pages].reshape(-1, D)
                vv = vh[pages].reshape(-1, D)
                for t in members:
                    keep = pos <= t
                    if not keep.any():
                        continue
                    qq = pb.q_rows(t, h)
                    s = (qq @ kk[keep].T) / math.sqrt(D)
                    m = s.max(axis=1)
                    e = np.exp(s - m[:, None])
                    partials.setdefault(t, []).append((m, e.sum(axis=1), e @ vv[keep]))
        for t, parts in partials.items():
            mm = np.max(np.stack([p[0] for p in parts]), axis=0)
            ll = sum(p[1] * np.exp(p[0] - mm) for p in parts)
            aa = sum(p[2] * np.exp(p[0] - mm)[:, None] for p in parts)
            out[t, h * G:(h + 1) * G] = aa / ll[:, None]
    return out
