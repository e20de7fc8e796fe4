"""Pins of the CPU greedy grouping (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle.greedy import group_head, group_ids, greedy_window

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "greedy_cases.json")


def _cases():
    return json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    sel = np.array(case["sel"], dtype=np.int32)[None]
    ids = group_ids(sel, case["N"], case["W"], case["g"])
    assert ids[0].tolist() == case["expected"]


def _brute(sel_h, N, W, g):
    """Independent implementation: boolean page matrix, explicit index loops."""
    T = sel_h.shape[0]
    mat = np.zeros((T, N), dtype=bool)
    for t in range(T):
        for u in sel_h[t]:
            if 0 <= u < N:
                mat[t, u] = True
    out = []
    for w0 in range(0, T, W):
        w1 = min(T, w0 + W)
        taken = np.zeros(T, dtype=bool)
        taken[:w0] = True
        taken[w1:] = True
        while not taken.all():
            seed = int(np.flatnonzero(~taken)[0])
            taken[seed] = True
            members = [seed]
            cover = mat[seed].copy()
            while len(members) < g and not taken.all():
                costs = np.where(taken, np.iinfo(np.int64).max,
                                 (mat & ~cover[None, :]).sum(axis=1))
                c = int(np.argmin(costs))            # argmin returns the first (lowest) index
                taken[c] = True
                members.append(c)
                cover |= mat[c]
            out.extend(members)
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(2, 65))
    W = int(rng.choice([4, 8, 16, 32]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    T = int(W * rng.integers(1, 4) - rng.integers(0, 3))
    S = int(rng.integers(1, 10))
    sel = rng.integers(-2, N + 2, size=(T, S)).astype(np.int32)
    if seed % 3 == 0:          # clustered supports make zero-cost ties common
        sel = (sel % 6).astype(np.int32)
    got = group_head(sel, N, W, g)
    assert np.array_equal(got, _brute(sel, N, W, g))


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    T, N, S, W, g = 96, 40, 6, 32, 8
    sel = rng.integers(-1, N, size=(2, T, S)).astype(np.int32)
    ids = group_ids(sel, N, W, g)
    for h in range(2):
        assert sorted(ids[h].tolist()) == list(range(T))          # a permutation
        for w0 in range(0, T, W):
            blk = ids[h, w0:w0 + W]
            assert blk.min() >= w0 and blk.max() < w0 + W          # stays in its window
            seen = set()
            for k in range(0, W, g):
                grp = blk[k:k + g].tolist()
                rest = [x for x in range(w0, w0 + W) if x not in seen]
                assert grp[0] == min(rest)                         # lowest unassigned seeds
                seen.update(grp)


def test_g1_is_identity_and_w_equals_g():
    rng = np.random.default_rng(7)
    sel = rng.integers(-1, 30, size=(1, 64, 5)).astype(np.int32)
    assert np.array_equal(group_ids(sel, 30, 16, 1)[0], np.arange(64))
    ids = group_ids(sel, 30, 8, 8)[0]
    for w0 in range(0, 64, 8):
        assert sorted(ids[w0:w0 + 8].tolist()) == list(range(w0, w0 + 8))
        assert ids[w0] == w0


def test_parallel_driver_matches_serial():
    rng = np.random.default_rng(3)
    sel = rng.integers(-1, 50, size=(3, 256, 7)).astype(np.int32)
    a = group_ids(sel, 50, 32, 8, workers=1)
    b = group_ids(sel, 50, 32, 8, workers=4)
    assert np.array_equal(a, b)
    part = group_ids(sel, 50, 32, 8, windows={1: [64, 192]})
    assert np.array_equal(part[1, 64:96], a[1, 64:96]) and np.array_equal(part[1, 192:224], a[1, 192:224])
    assert (part[0] == -1).all()


def test_greedy_window_direct():
    bits = [0b0011, 0b11100, 0b100011, 0b0010]
    assert greedy_window(bits, 2) == [0, 3, 1, 2]
