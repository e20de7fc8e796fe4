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


def test_tile_units_by_hand_and_brute_force():
    # one head, a group of 4 queries at G = 16: 64 rows in two 32-row tiles of 2 slots each
    sel = np.array([[[0, 1], [1, 2], [3, 3], [4, -1]]], dtype=np.int32)
    ids = np.array([[0, 1, 2, 3]], dtype=np.int32)
    # tile 0: queries 0, 1 -> {0, 1, 2}; tile 1: queries 2, 3 -> {3, 4}; the group union has 5
    assert bench.tile_units(sel, ids, 4, 16, N=8) == 5
    assert bench.tile_units(sel, ids, 4, 8, N=8) == 5         # one tile: the group union
    assert bench.union_stats(sel, ids, 4, N=8).sum() == 5
    assert bench.tile_units(np.array([[[0, 1], [0, 1], [0, 1], [0, 1]]], np.int32), ids, 4, 16, 8) == 4
    # random cases against a set-based count
    rng = np.random.default_rng(3)
    H, T, S, N = 2, 64, 5, 40
    sel = rng.integers(-1, N, size=(H, T, S)).astype(np.int32)
    ids = np.stack([rng.permutation(T) for _ in range(H)]).astype(np.int32)
    for g, G in [(8, 4), (8, 8), (16, 4), (5, 8), (3, 32), (7, 8)]:
        want = 0
        for h in range(H):
            for k0 in range(0, T, g):
                mem = ids[h, k0:k0 + g]
                for rt in range((g * G + 31) // 32):
                    pages = set()
                    for s in range(len(mem)):
                        if (32 * rt) // G <= s <= (32 * rt + 31) // G:
                            pages |= {int(u) for u in sel[h, mem[s]] if 0 <= u < N}
                    want += len(pages)
        assert bench.tile_units(sel, ids, g, G, N) == want, (g, G)


def test_recorded_traffic_per_workload_and_stale_hash(tmp_path, monkeypatch):
    # DRAM bytes come from the stored counter record only while its kernel hash matches the
    # current sources, and per workload; an unknown workload or a stale hash gives None
    import json
    rec = {"kernel_sha256_16": bench.kernel_hash(), "workload": "prefill_64k",
           "dram_bytes_per_launch": 5.0,
           "workloads": {"prefill_8k": {"dram_bytes_per_launch": 1.0},
                         "prefill_64k": {"dram_bytes_per_launch": 2.0}}}
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / "union_attn_counters.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: rec["kernel_sha256_16"])
    assert bench.recorded_traffic("prefill_8k") == 1.0
    assert bench.recorded_traffic("prefill_64k") == 2.0
    assert bench.recorded_traffic("prefill_32k") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.recorded_traffic("prefill_8k") is None


def test_stored_counters_match_the_current_kernel():
    # the committed counter record was taken on the current attention sources and build flags
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "union_attn_counters.json")))
    assert rec["kernel_sha256_16"] == bench.kernel_hash()
    for wl in ("prefill_8k", "prefill_32k", "prefill_64k", "prefill_64k_70b"):
        per = rec["workloads"][wl]
        assert per["dram_bytes_per_launch"] >= per["compulsory_bytes"] > 0
