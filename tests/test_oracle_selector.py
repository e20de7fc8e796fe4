"""Pins for the synthetic page selector oracle (oracle/selector.py).

The selector rule is a stand-in of our own (the pages take each query's page
selection as given); these tests pin the oracle against an exact-rational
brute force with an independent selection loop, invariants and constructed
cases, not against itself.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.fp8 import decode_bf16, decode_e4m3fn
from oracle.selector import fixed_pages, select, select_row


def _problem(T, Hq, Hkv, D, P, seed):
    N = T // P
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = torch.randn((T, Hq, D), generator=gen).to(torch.bfloat16)
    k = torch.randn((N, Hkv, P, D), generator=gen).to(torch.float8_e4m3fn)
    return (q.view(torch.int16).numpy().view(np.uint16), k.view(torch.uint8).numpy(),
            rng.uniform(0.05, 1.0, size=(2, N, Hkv)).astype(np.float32))


def _brute_row(q_bits, k_codes, scales, h, t, S, L, P):
    """Exact rational scores; the best remaining candidate is taken one at a time."""
    T, Hq, D = q_bits.shape
    G = Hq // k_codes.shape[1]
    p = t // P
    qv = decode_bf16(q_bits[t, h * G:(h + 1) * G])            # [G][D], exact binary values
    qs = [sum(Fraction(float(qv[j, d])) for j in range(G)) for d in range(D)]
    fixed = set([0] + [p - i for i in range(L) if p - i >= 0])
    score = {}
    for u in range(1, p + 1):
        if u in fixed:
            continue
        kv = decode_e4m3fn(k_codes[u, h])                      # [P][D]
        c = [sum(Fraction(float(kv[j, d])) for j in range(P)) for d in range(D)]
        score[u] = Fraction(float(scales[0, u, h])) * sum(a * b for a, b in zip(qs, c))
    chosen = []
    while len(fixed) + len(chosen) < S and score:
        best = None
        for u in sorted(score):                                # ascending: first max wins ties
            if best is None or score[u] > score[best]:
                best = u
        chosen.append(best)
        del score[best]
    row = sorted(fixed | set(chosen))
    return row + [-1] * (S - len(row))


@pytest.mark.parametrize("seed", range(3))
def test_matches_exact_brute_force(seed):
    T, Hq, Hkv, D, P, S, L = 64, 4, 2, 8, 4, 5, 2
    q, k, sc = _problem(T, Hq, Hkv, D, P, seed)
    got = select(q, k, sc, S, L, P)
    for h in range(Hkv):
        for t in range(0, T, 3):
            assert got[(h, t)].tolist() == _brute_row(q, k, sc, h, t, S, L, P), (h, t)


def test_invariants():
    T, Hq, Hkv, D, P, S, L = 256, 8, 2, 16, 8, 6, 2
    q, k, sc = _problem(T, Hq, Hkv, D, P, 7)
    got = select(q, k, sc, S, L, P)
    for (h, t), row in got.items():
        p = t // P
        valid = row[row >= 0]
        assert np.all(np.diff(valid) > 0)                       # ascending, no repeats
        assert valid.size == min(S, p + 1)                      # as many as exist, at most S
        assert np.all(row[valid.size:] == -1)
        assert valid.max() <= p and valid.min() == 0            # causal; the sink is kept
        assert set(fixed_pages(p, L)) <= set(valid.tolist())


def test_all_pages_when_they_fit():
    T, Hq, Hkv, D, P, S, L = 32, 2, 1, 8, 4, 8, 1
    q, k, sc = _problem(T, Hq, Hkv, D, P, 3)
    got = select(q, k, sc, S, L, P)
    for t in range(T):
        p = t // P
        assert got[(0, t)][: p + 1].tolist() == list(range(p + 1))


def test_scale_boost_and_ties():
    T, Hq, Hkv, D, P, S, L = 128, 2, 1, 8, 8, 3, 1          # one free slot per query
    q, k, sc = _problem(T, Hq, Hkv, D, P, 11)
    t = T - 1
    p = t // P
    qs = decode_bf16(q[t]).sum(axis=0)
    dots = [float(qs @ decode_e4m3fn(k[u, 0]).sum(axis=0)) for u in range(T // P)]
    u_pos = next(u for u in range(1, p - 1) if dots[u] > 0)
    boosted = sc.copy()
    boosted[0, u_pos, 0] = 1e6                                  # a huge positive score
    assert select(q, k, boosted, S, L, P, rows=[t])[(0, t)].tolist() == sorted({0, p, u_pos})
    # two identical pages tie exactly: the lower one is chosen
    k2, sc2 = k.copy(), boosted.copy()
    u_hi = next(u for u in range(p - 1, 0, -1) if u > u_pos)
    k2[u_hi], sc2[:, u_hi] = k2[u_pos], sc2[:, u_pos]
    assert select(q, k2, sc2, S, L, P, rows=[t])[(0, t)].tolist() == sorted({0, p, u_pos})
    # select_row itself: equal scores resolve to the lower page
    assert select_row(np.array([0.0, 1.0, 1.0, 0.5]), 3, 3, 1).tolist() == [0, 1, 3]
