"""Host-side logic of bench.py (no GPU): the one-GPU guard and the union/pair accounting."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_union_stats_counts_distinct_valid_pages():
    # one head, 6 queries, groups of 3 by the IDs [5, 0, 2 | 1, 3, 4]
    sel = np.array([[[0, 1, -1], [0, 2, 2], [3, -1, 9], [1, 1, 1], [4, 0, -1], [0, 5, 1]]],
                   dtype=np.int32)
    ids = np.array([[5, 0, 2, 1, 3, 4]], dtype=np.int32)
    got = bench.union_stats(sel, ids, 3, N=8)
    # group 0: queries 5, 0, 2 -> {0, 5, 1} | {0, 1} | {3} (9 is out of range) = {0, 1, 3, 5}
    # group 1: queries 1, 3, 4 -> {0, 2} | {1} | {4, 0} = {0, 1, 2, 4}
    assert got.tolist() == [[4, 4]]
    # a ragged last group (g = 4: groups of 4 and 2)
    got4 = bench.union_stats(sel, ids, 4, N=8)
    assert got4.tolist() == [[5, 3]]


def test_pair_entries_adjacent_and_table():
    sel = np.array([[[0, 1, 2, -1], [2, 3, 5, 9]]], dtype=np.int32)
    assert bench.pair_entries(sel, None, 6) == 2.0
    pairs = np.full((1, 6, 2), -1, np.int32)
    pairs[0, :3] = [[0, 2], [1, 3], [4, 5]]
    assert bench.pair_entries(sel, pairs, 6) == 2.5
