"""Direct KV-page union (the pages' complementary design study), in fp64.

The pages contrast query groups with a direct KV-page union that studies
non-local reuse against its reduction cost ("PageWeaver: KV-Guided Query
Unions for Sparse Attention", Abstract); it works on disjoint page pairs and
uses the full membership of each page to form common and exclusive query lists
(AI Radio episode on the paper, section "Paper summary").  Unlike the query
union it produces one partial output per (query, page pair), so the per-query
results have to be merged afterwards.

Readings taken: pages are paired either by ID as (2k, 2k+1) or by affinity
(below); the full membership of a pair is every query of that KV head that
selected either page; the common list holds the queries that selected both, the
exclusive lists those that selected exactly one of them; each (query, Q head,
pair) partial is (m, l, acc) over the query's own visible keys in the pair;
partials are merged by log-sum-exp.  The merged result is the same O as
``oracle.attention`` for any partition of the pages into pairs (only the order
of the floating-point work differs).

Affinity pairs (the tuned variant of the design study): pages that many
queries select together share more common-list entries, so pairs are chosen by
co-selection.  co[u][v] counts the queries of the KV head whose support holds
both u and v; the pairing is the greedy matching on the edges co > 0 taken in
the order (larger count first, then lower first page, then lower second page):
an edge joins the matching when both its pages are still free.  Unmatched
pages stay single.  Pairs are numbered by their lower page.
TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .attention import Problem

Pair = Tuple[int, int]       # (lower page, higher page or -1 for a single page)


def adjacent_pairs(N: int) -> List[Pair]:
    """Pairs (2k, 2k+1) by page ID; an odd last page stays single."""
    return [(2 * k, 2 * k + 1 if 2 * k + 1 < N else -1) for k in range((N + 1) // 2)]


def coselection(sel_h: np.ndarray, N: int) -> np.ndarray:
    """co[u][v] = number of queries whose support (valid entries of its row) holds u and v;
    the diagonal is 0.  int64 [N][N].  The count matrix is A^T A for the query x page
    membership matrix A, formed with a float matmul (exact: counts are far below 2^24)."""
    T = sel_h.shape[0]
    A = np.zeros((T, N), dtype=np.float32)
    rows, cols = np.nonzero((sel_h >= 0) & (sel_h < N))
    A[rows, sel_h[rows, cols]] = 1.0
    co = np.rint(A.T @ A).astype(np.int64)
    np.fill_diagonal(co, 0)
    return co


def affinity_pairs(sel_h: np.ndarray, N: int) -> List[Pair]:
    """Greedy co-selection matching of one KV head's pages, as described above."""
    co = coselection(sel_h, N)
    u, v = np.nonzero(np.triu(co, 1) > 0)
    order = np.lexsort((v, u, -co[u, v]))          # count desc, then u, then v
    mate = np.full(N, -1, dtype=np.int64)
    for i in order:
        a, b = int(u[i]), int(v[i])
        if mate[a] < 0 and mate[b] < 0:
            mate[a], mate[b] = b, a
    return pairs_from_mates(mate)


def pairs_from_mates(mate: np.ndarray) -> List[Pair]:
    """Pair list (numbered by lower page) from a mate array (-1 = single)."""
    N = mate.shape[0]
    return [(a, int(mate[a]) if mate[a] > a else -1) for a in range(N)
            if mate[a] < 0 or mate[a] > a]


def matching_weight(co: np.ndarray, pairs: Sequence[Pair]) -> int:
    """Sum of co[a][b] over the pairs (singles add 0): the (query, pair) entries the pairing
    saves against one entry per selected page."""
    return int(sum(co[a, b] for a, b in pairs if b >= 0))


def max_coselection_pairs(sel_h: np.ndarray, N: int) -> List[Pair]:
    """A maximum co-selection matching of one KV head's pages: pairs of distinct pages, each
    page in at most one pair, maximising the sum of co[u][v] over the pairs (the reading of
    "max co-selection matching"; unmatched pages stay single).

    Written as the matching integer program, one 0/1 variable per edge with co > 0, one
    "at most one edge per page" row per page, solved exactly (HiGHS branch and bound with
    zero optimality gap).  Several matchings can reach the maximum: only the weight is unique.
    """
    from scipy.optimize import Bounds, LinearConstraint, milp
    from scipy.sparse import csr_matrix
    co = coselection(sel_h, N)
    u, v = np.nonzero(np.triu(co, 1) > 0)
    if u.size == 0:
        return pairs_from_mates(np.full(N, -1, dtype=np.int64))
    E = u.size
    rows = np.concatenate([u, v])
    cols = np.concatenate([np.arange(E), np.arange(E)])
    A = csr_matrix((np.ones(2 * E), (rows, cols)), shape=(N, E))
    res = milp(c=-co[u, v].astype(np.float64), constraints=LinearConstraint(A, 0, 1),
               integrality=np.ones(E), bounds=Bounds(0, 1),
               options={"mip_rel_gap": 0.0, "presolve": True})
    if res.status != 0:
        raise RuntimeError(f"matching program not solved: {res.message}")
    x = np.rint(res.x).astype(np.int64)
    assert np.all(np.abs(res.x - x) < 1e-6) and np.all(A @ x <= 1)
    mate = np.full(N, -1, dtype=np.int64)
    for e in np.nonzero(x)[0]:
        mate[u[e]], mate[v[e]] = v[e], u[e]
    return pairs_from_mates(mate)


def pair_lists(pb: Problem, h: int, pairs: Optional[Sequence[Pair]] = None
               ) -> Dict[int, Dict[str, List[int]]]:
    """pair k -> {'common': [...], 'only_first': [...], 'only_second': [...]}, sorted query IDs."""
    pairs = adjacent_pairs(pb.N) if pairs is None else pairs
    where = {}
    for k, (a, b) in enumerate(pairs):
        where[a] = (k, 0)
        if b >= 0:
            where[b] = (k, 1)
    lists: Dict[int, Dict[str, List[int]]] = {}
    for t in range(pb.T):
        hit: Dict[int, set] = {}
        for u in pb.support(h, t).tolist():
            k, pos = where[u]
            hit.setdefault(k, set()).add(pos)
        for k in sorted(hit):
            kind = "common" if len(hit[k]) == 2 else ("only_first" if 0 in hit[k] else "only_second")
            lists.setdefault(k, {"common": [], "only_first": [], "only_second": []})[kind].append(t)
    return lists


def dense_union(pb: Problem, pairing: Optional[Dict[int, Sequence[Pair]]] = None) -> np.ndarray:
    """O as fp64 [T][H_q][D] via per-pair partials and a log-sum-exp merge.

    ``pairing`` maps KV head -> its pairs (default: adjacent pairs for every head)."""
    G, D, P = pb.G, pb.D, pb.P
    out = np.zeros((pb.T, pb.H_q, D))
    for h in range(pb.H_kv):
        pairs = adjacent_pairs(pb.N) if pairing is None else pairing[h]
        kh, vh = pb.k_hat(h), pb.v_hat(h)
        partials: Dict[int, list] = {}
        for k, kinds in sorted(pair_lists(pb, h, pairs).items()):
            a, b = pairs[k]
            for kind, members in kinds.items():
                pages = {"common": [a, b], "only_first": [a], "only_second": [b]}[kind]
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
