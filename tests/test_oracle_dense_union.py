"""Pins of the direct KV-page union oracle (CPU only).

The merged result is pinned to the per-query attention oracle for adjacent and
affinity pairs.  The affinity matching is pinned by an independent brute force
(co-selection counted with Python sets, the matching built by repeatedly taking
the best remaining edge), by the certificate that characterises the greedy
matching of a strict edge order (every unmatched edge has an endpoint matched
by an earlier edge), and by a hand-worked case.
"""
import itertools

import numpy as np
import pytest

from oracle.attention import Problem, attention
from oracle.dense_union import adjacent_pairs, affinity_pairs, coselection, dense_union, pair_lists
from tests.oracle_helpers import tiny_problem


def _pb(inp):
    return Problem(inp["q_bits"], inp["k_codes"], inp["v_codes"], inp["scales"], inp["sel_pages"])


@pytest.mark.parametrize("seed", [0, 1])
def test_pairwise_partials_merge_to_the_per_query_result(seed):
    inp = tiny_problem(T=128, P=16, Hq=4, Hkv=2, D=16, S=5, seed=seed)
    pb = _pb(inp)
    np.testing.assert_allclose(dense_union(pb), attention(pb), rtol=0, atol=1e-12)


def test_pair_lists_partition_membership():
    inp = tiny_problem(T=96, P=16, S=4, seed=3)
    pb = _pb(inp)
    for h in range(2):
        lists = pair_lists(pb, h)
        for k, kinds in lists.items():
            for kind, members in kinds.items():
                assert members == sorted(members)
                for t in members:
                    sup = set(pb.support(h, t).tolist())
                    e, o = 2 * k in sup, 2 * k + 1 in sup
                    assert (kind == "common") == (e and o)
                    assert (kind == "only_first") == (e and not o)
                    assert (kind == "only_second") == (o and not e)
        # every (query, selected page) lands in exactly one list of its pair
        for t in range(pb.T):
            for u in pb.support(h, t).tolist():
                hits = [kind for kind, m in lists[u // 2].items() if t in m]
                assert len(hits) == 1


def _brute_pairs(sel_h, N):
    """Independent brute force: set-based counts; repeatedly take the best free edge."""
    sup = [set(int(u) for u in row if 0 <= u < N) for row in sel_h]
    co = {}
    for a, b in itertools.combinations(range(N), 2):
        c = sum(1 for s in sup if a in s and b in s)
        if c:
            co[(a, b)] = c
    free = set(range(N))
    pairs = []
    while True:
        best = None
        for (a, b), c in co.items():
            if a in free and b in free:
                if best is None or c > best[0] or (c == best[0] and (a, b) < best[1]):
                    best = (c, (a, b))
        if best is None:
            break
        a, b = best[1]
        pairs.append((a, b))
        free -= {a, b}
    pairs += [(a, -1) for a in free]
    return sorted(pairs)


@pytest.mark.parametrize("seed", range(4))
def test_affinity_pairs_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, N, S = 40, 12, 4
    sel = rng.integers(-2, N + 1, size=(T, S)).astype(np.int32)
    sel[::4] = sel[::4] % 3                       # repeated rows: many equal counts (ties)
    assert affinity_pairs(sel, N) == _brute_pairs(sel, N)


@pytest.mark.parametrize("seed", range(3))
def test_affinity_pairs_greedy_certificate(seed):
    # a partition of the pages whose every unmatched edge (co > 0) has an endpoint
    # matched by an edge earlier in the order is the greedy matching, and only it
    inp = tiny_problem(T=512, P=8, Hq=2, Hkv=1, D=8, S=7, seed=seed)
    sel, N = inp["sel_pages"][0], inp["k_codes"].shape[0]
    pairs = affinity_pairs(sel, N)
    co = coselection(sel, N)
    pages = sorted([a for a, _ in pairs] + [b for _, b in pairs if b >= 0])
    assert pages == list(range(N))                           # a partition
    assert [a for a, _ in pairs] == sorted(a for a, _ in pairs)
    mate = {}
    for a, b in pairs:
        assert b == -1 or (a < b and co[a, b] > 0)
        if b >= 0:
            mate[a], mate[b] = b, a
    key = lambda a, b: (-co[a, b], min(a, b), max(a, b))
    for a in range(N):
        for b in range(a + 1, N):
            if co[a, b] == 0 or mate.get(a) == b:
                continue
            dominated = any(x in mate and key(x, mate[x]) < key(a, b) for x in (a, b))
            assert dominated, (a, b)
    assert any(b >= 0 for _, b in pairs)


def test_affinity_pairs_hand_case():
    # pages 0..5; queries: four select {0, 1, 2}, three select {3, 4}, two select {2, 5}
    # counts: (0,1)=4 (0,2)=4 (1,2)=4 (3,4)=3 (2,5)=2, all others 0.
    # greedy: (0,1) first (count 4, lowest pages), then (0,2)/(1,2) are blocked,
    # (3,4) next, then (2,5).  Every page is paired.
    rows = [[0, 1, 2]] * 4 + [[3, 4, -1]] * 3 + [[2, 5, -1]] * 2
    sel = np.array(rows, dtype=np.int32)
    assert affinity_pairs(sel, 6) == [(0, 1), (2, 5), (3, 4)]
    # a page nobody selects stays single; the count matrix ignores -1 and out-of-range IDs
    sel2 = np.array([[0, 1, 7], [0, 1, -3]], dtype=np.int32)
    assert affinity_pairs(sel2, 3) == [(0, 1), (2, -1)]
    assert coselection(sel2, 3)[0, 1] == 2
    co = coselection(sel, 6)
    assert (np.diag(co) == 0).all() and (co == co.T).all()
    assert co[0, 1] == co[0, 2] == co[1, 2] == 4 and co[3, 4] == 3 and co[2, 5] == 2 and co.sum() == 2 * 17


def test_adjacent_pairs_shape():
    assert adjacent_pairs(5) == [(0, 1), (2, 3), (4, -1)]
    assert adjacent_pairs(4) == [(0, 1), (2, 3)]


@pytest.mark.parametrize("seed", [0, 1])
def test_affinity_partials_merge_to_the_per_query_result(seed):
    inp = tiny_problem(T=256, P=8, Hq=4, Hkv=2, D=16, S=6, seed=seed)
    pb = _pb(inp)
    pairing = {h: affinity_pairs(inp["sel_pages"][h], pb.N) for h in range(pb.H_kv)}
    assert any(b >= 0 and b != a + 1 for pr in pairing.values() for a, b in pr)   # not adjacent
    np.testing.assert_allclose(dense_union(pb, pairing), attention(pb), rtol=0, atol=1e-12)


# ---- the maximum co-selection matching (exact integer program) ----------------------------

def _brute_max_weight(co, N):
    """Best total weight over every matching of N pages, by exhaustive recursion."""
    best = 0

    def rec(free, w):
        nonlocal best
        best = max(best, w)
        if len(free) < 2:
            return
        a = free[0]
        rest = free[1:]
        rec(rest, w)                                  # a stays single
        for i, b in enumerate(rest):
            if co[a][b] > 0:
                rec(rest[:i] + rest[i + 1:], w + co[a][b])
    rec(list(range(N)), 0)
    return best


def _is_matching(pairs, N):
    seen = [p for pr in pairs for p in pr if p >= 0]
    return sorted(seen) == list(range(N)) and all(b == -1 or a < b for a, b in pairs)


@pytest.mark.parametrize("seed", range(6))
def test_max_matching_equals_exhaustive_search(seed):
    from oracle.dense_union import matching_weight, max_coselection_pairs
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(4, 10))
    T = 40
    sel_h = np.full((T, 4), -1, dtype=np.int32)
    for t in range(T):
        k = int(rng.integers(1, 5))
        sel_h[t, :k] = rng.choice(N, size=k, replace=False)
    # set-based counts, independent of coselection()
    sup = [set(int(u) for u in row if 0 <= u < N) for row in sel_h]
    co = [[sum(1 for s in sup if a in s and b in s) if a != b else 0 for b in range(N)]
          for a in range(N)]
    pairs = max_coselection_pairs(sel_h, N)
    assert _is_matching(pairs, N)
    assert matching_weight(np.array(co), pairs) == _brute_max_weight(co, N)


def test_max_matching_beats_greedy_on_a_path():
    # path 0-1-2-3 with co = 2, 3, 2: the greedy takes (1, 2) (weight 3), the maximum
    # matching takes (0, 1) and (2, 3) (weight 4)
    from oracle.dense_union import affinity_pairs, matching_weight, max_coselection_pairs
    rows = [[0, 1]] * 2 + [[1, 2]] * 3 + [[2, 3]] * 2
    sel_h = np.array([r + [-1] for r in rows], dtype=np.int32)
    co = coselection(sel_h, 4)
    assert affinity_pairs(sel_h, 4) == [(0, -1), (1, 2), (3, -1)]
    assert max_coselection_pairs(sel_h, 4) == [(0, 1), (2, 3)]
    assert matching_weight(co, affinity_pairs(sel_h, 4)) == 3
    assert matching_weight(co, max_coselection_pairs(sel_h, 4)) == 4


@pytest.mark.parametrize("seed", [0, 1])
def test_greedy_is_within_half_of_the_maximum(seed):
    # the greedy matching of a weight order is a 1/2-approximation of the maximum weight
    from oracle.dense_union import affinity_pairs, matching_weight, max_coselection_pairs
    inp = tiny_problem(T=256, P=16, S=6, seed=seed)
    for h in range(2):
        sel_h = inp["sel_pages"][h]
        co = coselection(sel_h, 16)
        g = matching_weight(co, affinity_pairs(sel_h, 16))
        m = matching_weight(co, max_coselection_pairs(sel_h, 16))
        assert _is_matching(max_coselection_pairs(sel_h, 16), 16)
        assert m >= g >= m / 2


def test_max_matching_merges_to_the_per_query_result():
    from oracle.dense_union import max_coselection_pairs
    inp = tiny_problem(T=128, P=16, Hq=4, Hkv=2, D=16, S=5, seed=4)
    pb = _pb(inp)
    pairing = {h: max_coselection_pairs(inp["sel_pages"][h], pb.N) for h in range(2)}
    np.testing.assert_allclose(dense_union(pb, pairing), attention(pb), rtol=0, atol=1e-12)
