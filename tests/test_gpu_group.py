"""pw_group on the GPU against the CPU greedy oracle: bit-exact query IDs."""
import time

import numpy as np
import pytest
import torch

from query_union_paged_amd import synth
from oracle.greedy import group_ids
from tests.gpu_common import WORKERS, host_inputs, log

pytestmark = pytest.mark.gpu


def _pw():
    from query_union_paged_amd import pageweaver
    return pageweaver


def _gpu_ids(sel_np, N, P, W, g, H_q=None, D=128):
    pw = _pw()
    H, T, S = sel_np.shape
    shp = pw.shape(T, H_q or H, H, D, P, N, S)
    sel = torch.from_numpy(sel_np).cuda()
    ids = pw.pw_group(shp, sel, W, g)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_group_ids_bit_exact(name):
    wl = synth.WORKLOADS[name]
    log(f"[case] pw_group {name} W={wl.W} g={wl.g}")
    sel = host_inputs(name)["sel_pages"]
    got = _gpu_ids(sel, wl.N, wl.P, wl.W, wl.g, wl.H_q, wl.D)
    t0 = time.time()
    ref = group_ids(sel, wl.N, wl.W, wl.g, workers=WORKERS)
    log(f"[oracle] greedy {name}: {time.time() - t0:.1f}s on {WORKERS} processes")
    assert np.array_equal(got, ref), f"{(got != ref).sum()} IDs differ"


@pytest.mark.parametrize("W,g", [(32, 1), (33, 3), (64, 8), (96, 8), (128, 4), (256, 8), (200, 5), (256, 2),
                                 (64, 16), (256, 16), (80, 10), (96, 12)])
def test_group_windows_and_sizes(W, g):
    # random supports over N = 256 pages, including ragged last windows and groups
    log(f"[case] pw_group random W={W} g={g}")
    rng = np.random.default_rng(W * 10 + g)
    T, P, S = 1024, 4, 12
    N = T // P
    sel = rng.integers(-3, N + 3, size=(2, T, S)).astype(np.int32)
    sel[:, ::3] %= 20        # clustered rows: many equal-cost ties
    got = _gpu_ids(sel, N, P, W, g)
    ref = group_ids(sel, N, W, g, workers=WORKERS)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("W,g", [(384, 8), (512, 8), (768, 4), (1024, 8), (960, 12), (300, 5),
                                 (1024, 1), (640, 16)])
def test_group_wide_windows(W, g):
    # several waves share one window (W > 256); T = 2048 gives full and ragged windows
    log(f"[case] pw_group wide window W={W} g={g}")
    rng = np.random.default_rng(W * 7 + g)
    T, P, S = 2048, 4, 12
    N = T // P
    sel = rng.integers(-3, N + 3, size=(2, T, S)).astype(np.int32)
    sel[:, ::3] %= 20
    sel[:, 1::5] = sel[:, 1::5] % 700      # words past 512 pages are never active: fewer words
    got = _gpu_ids(sel, N, P, W, g)
    ref = group_ids(sel, N, W, g, workers=WORKERS)
    assert np.array_equal(got, ref), f"{(got != ref).sum()} IDs differ"


def test_group_wide_window_64k_sample():
    # W = 1024 at the 64K workload's shape; two windows per head against the oracle
    wl = synth.WORKLOADS["prefill_64k"]
    W, g = 1024, 8
    log(f"[case] pw_group prefill_64k W={W} g={g} (sampled windows)")
    sel = host_inputs("prefill_64k")["sel_pages"]
    got = _gpu_ids(sel, wl.N, wl.P, W, g, wl.H_q, wl.D)
    starts = {h: [0, (wl.T // W - 1) * W] if h % 2 == 0 else [(wl.T // W // 2) * W]
              for h in range(wl.H_kv)}
    ref = group_ids(sel, wl.N, W, g, workers=WORKERS, windows=starts)
    for h, st in starts.items():
        for w0 in st:
            assert np.array_equal(got[h, w0:w0 + W], ref[h, w0:w0 + W]), (h, w0)
    assert all(np.array_equal(np.sort(r), np.arange(wl.T)) for r in got)


@pytest.mark.parametrize("N", [64, 100, 1024])
def test_group_page_counts(N):
    log(f"[case] pw_group N={N}")
    rng = np.random.default_rng(N)
    P = 16
    T = N * P
    sel = rng.integers(0, N, size=(1, T, 6)).astype(np.int32)
    got = _gpu_ids(sel, N, P, 64, 8)
    ref = group_ids(sel, N, 64, 8, workers=WORKERS)
    assert np.array_equal(got, ref)


def test_group_golden_cases():
    import json
    import os
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "greedy_cases.json")))
    for case in doc["cases"]:
        log(f"[case] pw_group golden {case['name']}")
        sel = np.array(case["sel"], dtype=np.int32)
        T, N, W, g = sel.shape[0], case["N"], case["W"], case["g"]
        # The ABI needs T == N_pages * P.  Pad with empty queries only when the
        # padding forms windows of its own, so the real windows are unchanged.
        if T % N == 0:
            n_abi, p_abi = N, T // N
        elif T % W == 0 and N >= T:
            n_abi, p_abi = N, 1
        else:
            assert sel.max() < T
            n_abi, p_abi = T, 1
        t_abi = n_abi * p_abi
        full = np.full((1, t_abi, sel.shape[1]), -1, dtype=np.int32)
        full[0, :T] = sel
        got = _gpu_ids(full, n_abi, p_abi, W, g)
        assert got[0, :T].tolist() == case["expected"], case["name"]


def test_check_ids_counts():
    # permutations give 0; out-of-range entries and repeats are counted per KV head
    from query_union_paged_amd import pageweaver as pw
    log("[case] pw_check_ids")
    wl = synth.WORKLOADS["prefill_8k"]
    sel = torch.from_numpy(host_inputs("prefill_8k")["sel_pages"]).cuda()
    shp = pw.shape(*wl.shape_tuple())
    ids = pw.pw_group(shp, sel, wl.W, wl.g)
    assert pw.pw_check_ids(shp, ids).cpu().tolist() == [0] * wl.H_kv
    bad = ids.clone()
    bad[1, 5] = bad[1, 6]            # one repeat
    bad[3, 0] = -1                   # out of range
    bad[3, 1] = wl.T                 # out of range
    bad[3, 2] = bad[3, 3] = bad[3, 4]   # two repeats of one ID
    got = pw.pw_check_ids(shp, bad).cpu().numpy()
    b = bad.cpu().numpy()
    want = [int(((r < 0) | (r >= wl.T)).sum()) + int(((r >= 0) & (r < wl.T)).sum()) -
            len(set(r[(r >= 0) & (r < wl.T)].tolist())) for r in b]
    assert got.tolist() == want == [0, 1, 0, 4, 0, 0, 0, 0]


def _union_sizes(sel_np, ids, N, g):
    """Distinct valid pages of every group's members, numpy, [H][ceil(T / g)]."""
    H, T, _ = sel_np.shape
    ng = -(-T // g)
    out = np.zeros((H, ng), np.int64)
    for h in range(H):
        for k in range(ng):
            rows = sel_np[h, ids[h, k * g:(k + 1) * g]]
            out[h, k] = len(np.unique(rows[(rows >= 0) & (rows < N)]))
    return out


@pytest.mark.parametrize("case", ["prefill_8k", "rand256", "rand512_ragged", "wide1024"])
def test_group_order(case):
    # pw_group_ordered: the same IDs as pw_group, and per KV head and block of groups the block's
    # groups by ascending union size with equal sizes in index order (checked against sizes
    # counted here with numpy)
    pw = _pw()
    log(f"[case] pw_group_ordered {case}")
    if case == "prefill_8k":
        wl = synth.WORKLOADS[case]
        sel, N, P, W, g, Hq = host_inputs(case)["sel_pages"], wl.N, wl.P, wl.W, wl.g, wl.H_q
    else:
        rng = np.random.default_rng(len(case))
        T, P = {"rand256": (1024, 4), "rand512_ragged": (1020, 2), "wide1024": (2048, 4)}[case]
        N = T // P
        W, g = {"rand256": (64, 8), "rand512_ragged": (300, 5), "wide1024": (1024, 8)}[case]
        sel = rng.integers(-3, N + 3, size=(2, T, 12)).astype(np.int32)
        sel[:, ::3] %= 24                    # clustered rows: many groups of equal union size
        # G = 16 makes a group of 8 four waves: blocks of 64 groups (two per head here)
        Hq = {"rand256": 32, "rand512_ragged": 8, "wide1024": 2}[case]
    H, T, S = sel.shape
    shp = pw.shape(T, Hq, H, 128, P, N, S)
    sel_d = torch.from_numpy(sel).cuda()
    ids_plain = pw.pw_group(shp, sel_d, W, g)
    ids, order = pw.pw_group_ordered(shp, sel_d, W, g)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_plain)
    ids_np, order_np = ids.cpu().numpy(), order.cpu().numpy()
    sizes = _union_sizes(sel, ids_np, N, g)
    ng = sizes.shape[1]
    block = max(1, 256 // -(-g * (Hq // H) // 32))         # groups run at once on one XCD
    for h in range(H):
        want = []
        for b0 in range(0, ng, block):                      # blocks in index order
            idx = np.arange(b0, min(ng, b0 + block))
            want += list(idx[np.lexsort((idx, sizes[h, idx]))])   # by size, then by index
        assert np.array_equal(order_np[h], np.array(want)), f"head {h}"
    log(f"[parity] {case}: {ng} groups per head in blocks of {block}, union sizes "
        f"{sizes.min()}..{sizes.max()}")
