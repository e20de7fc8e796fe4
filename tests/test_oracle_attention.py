"""Pins of the fp64 attention oracle (CPU only)."""

import numpy as np
import pytest
import torch

from oracle.attention import (Problem, attention, attention_groupwise, attention_pairs,
                              attention_pairs_parallel, attention_query)
from oracle.greedy import group_ids
from tests.oracle_helpers import tiny_problem, torch_dense_reference


def _pb(inp):
    return Problem(inp["q_bits"], inp["k_codes"], inp["v_codes"], inp["scales"], inp["sel_pages"])


def test_all_pages_selected_is_full_causal_attention():
    # every page selected: the support reduces to plain causal attention
    T, P, Hkv = 64, 16, 2
    N = T // P
    sel = np.tile(np.arange(N, dtype=np.int32), (Hkv, T, 1))
    inp = tiny_problem(T=T, P=P, Hkv=Hkv, S=N, sel=sel, seed=1)
    ours = attention(_pb(inp))
    qb, kc, vc, sc = inp["q_bits"], inp["k_codes"], inp["v_codes"], inp["scales"]
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).double()
    k = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * torch.from_numpy(sc[0]).double()[:, :, None, None]
    v = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * torch.from_numpy(sc[1]).double()[:, :, None, None]
    k = k.permute(1, 0, 2, 3).reshape(Hkv, T, -1).repeat_interleave(2, dim=0)
    v = v.permute(1, 0, 2, 3).reshape(Hkv, T, -1).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q.transpose(0, 1), k, v, is_causal=True)
    np.testing.assert_allclose(ours, ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_subset_matches_masked_sdpa(seed):
    inp = tiny_problem(T=96, P=16, Hq=6, Hkv=2, D=8, S=3, seed=seed)
    sel = inp["sel_pages"]
    Hkv, T, _ = sel.shape
    P = 16
    allowed = np.zeros((Hkv, T, T), dtype=bool)
    for h in range(Hkv):
        for t in range(T):
            for u in sel[h, t]:
                if u >= 0:
                    allowed[h, t, u * P:(u + 1) * P] = True
    allowed &= np.tril(np.ones((T, T), dtype=bool))[None]
    ref = torch_dense_reference(inp, allowed)
    np.testing.assert_allclose(attention(_pb(inp)), ref, rtol=0, atol=1e-12)


def test_set_semantics_of_selection_rows():
    # repeats, -1 and out-of-range entries are empty slots; order is irrelevant
    inp = tiny_problem(T=64, P=16, S=4, seed=5)
    base = attention(_pb(inp))
    N = 4
    rng = np.random.default_rng(0)
    sel = inp["sel_pages"]
    wide = np.full(sel.shape[:2] + (sel.shape[2] + 5,), -1, dtype=np.int32)
    for h in range(sel.shape[0]):
        for t in range(sel.shape[1]):
            row = [int(u) for u in sel[h, t] if u >= 0]
            row = row + row[:1] + [-1, N, N + 7, -9]
            rng.shuffle(row)
            wide[h, t, :len(row)] = row
    np.testing.assert_array_equal(attention(_pb(dict(inp, sel_pages=wide))), base)


def test_closed_forms():
    inp = tiny_problem(T=48, P=16, Hq=2, Hkv=1, D=8, S=3, seed=9)
    pb = _pb(inp)
    # t = 0 sees exactly key 0 of page 0 (page 0 is its only visible page)
    v00 = pb.v_hat(0)[0, 0]
    o = attention_query(pb, 0, 0)
    np.testing.assert_allclose(o, np.tile(v00, (2, 1)), rtol=0, atol=1e-15)
    # Q = 0: uniform weights, O = mean of the visible V rows
    inp0 = dict(inp, q_bits=np.zeros_like(inp["q_bits"]))
    pb0 = _pb(inp0)
    for t in [5, 17, 33, 47]:
        sup = sorted({int(u) for u in inp["sel_pages"][0, t] if u >= 0})
        rows = [pb0.v_hat(0)[u, c] for u in sup for c in range(16) if u * 16 + c <= t]
        np.testing.assert_allclose(attention_query(pb0, 0, t), np.tile(np.mean(rows, axis=0), (2, 1)),
                                   rtol=0, atol=1e-13)
    # constant V (one code, one scale): O equals that constant
    inpc = dict(inp, v_codes=np.full_like(inp["v_codes"], 0x3C),
                scales=np.stack([inp["scales"][0], np.full_like(inp["scales"][1], 0.5)]))
    np.testing.assert_allclose(attention(_pb(inpc)), 0.75, rtol=0, atol=1e-14)


def test_empty_support_gives_zero():
    inp = tiny_problem(T=32, P=16, S=2, seed=4)
    sel = inp["sel_pages"].copy()
    sel[0, 20] = -1
    sel[1, 3] = [7, 9]        # out of range only
    o = attention(_pb(dict(inp, sel_pages=sel)))
    assert np.all(o[20, 0:2] == 0) and np.all(o[3, 2:4] == 0)


def test_query_order_and_parallel_driver():
    inp = tiny_problem(T=128, P=16, S=4, seed=11)
    pb = _pb(inp)
    pairs = [(h, t) for h in range(2) for t in range(128)]
    base = attention_pairs(pb, pairs)
    perm = np.random.default_rng(1).permutation(len(pairs))
    shuffled = attention_pairs(pb, [pairs[i] for i in perm])
    np.testing.assert_array_equal(shuffled, base[perm])
    par = attention_pairs_parallel(pb, [pairs[i] for i in perm], workers=3)
    np.testing.assert_array_equal(par, base[perm])


@pytest.mark.parametrize("mode", ["identity", "greedy", "random"])
def test_groupwise_union_equals_per_query(mode):
    inp = tiny_problem(T=128, P=16, Hq=4, Hkv=2, D=16, S=4, seed=21)
    pb = _pb(inp)
    T, g, W = 128, 8, 32
    if mode == "identity":
        ids = np.tile(np.arange(T, dtype=np.int32), (2, 1))
    elif mode == "greedy":
        ids = group_ids(inp["sel_pages"], T // 16, W, g)
    else:
        rng = np.random.default_rng(2)
        ids = np.stack([rng.permutation(T) for _ in range(2)]).astype(np.int32)
    np.testing.assert_allclose(attention_groupwise(pb, ids, g), attention(pb), rtol=0, atol=1e-12)
