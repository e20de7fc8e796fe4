"""Pins of the direct KV-page union oracle (CPU only)."""
import numpy as np
import pytest

from oracle.attention import Problem, attention
from oracle.dense_union import dense_union, pair_lists
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
                    assert (kind == "only_even") == (e and not o)
                    assert (kind == "only_odd") == (o and not e)
        # every (query, selected page) lands in exactly one list of its pair
        for t in range(pb.T):
            for u in pb.support(h, t).tolist():
                hits = [kind for kind, m in lists[u // 2].items() if t in m]
                assert len(hits) == 1
