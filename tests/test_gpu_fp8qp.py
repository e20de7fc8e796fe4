"""pw_union_attention_tiled_fp8qp (Q and P in e4m3fn) on the GPU against its fp64 model
(oracle.lowp), and its distance from the exact attention (oracle.attention)."""
import numpy as np
import pytest
import torch

from query_union_paged_amd import synth
from tests.fp8qp_gate import assert_close_lowp, model_rows
from tests.gpu_common import (TOL_MEAN, errors, gpu_rows, host_inputs, log, oracle_rows,
                              sample_pairs, window_sample_pairs)
from tests.oracle_helpers import tiny_problem

pytestmark = pytest.mark.gpu

def _pw():
    from query_union_paged_amd import pageweaver
    return pageweaver


def _shape(inp):
    pw = _pw()
    T, Hq, D = inp["q_bits"].shape
    N, Hkv, P, _ = inp["k_codes"].shape
    return pw.shape(T, Hq, Hkv, D, P, N, inp["sel_pages"].shape[2])


def _run(inp, g, ids=None, W=None, order=None, dev=None):
    """Upload (unless given), IDs (search, or given), tile, then the FP8 variant."""
    pw = _pw()
    dev = dev or pw.to_device(inp)
    shp = _shape(inp)
    if ids is None:
        ids = pw.pw_group(shp, dev["sel_pages"], W, g)
    elif isinstance(ids, np.ndarray):
        ids = torch.from_numpy(ids).cuda()
    ws = pw.pw_tile_kv(shp, dev["k_codes"], dev["v_codes"], dev["scales"])
    O = pw.pw_union_attention_tiled_fp8qp(shp, dev["q_bits"], dev["sel_pages"], ids, g, ws,
                                          group_order=order)
    torch.cuda.synchronize()
    return O, ids, dev


def _identity(T, Hkv):
    return np.tile(np.arange(T, dtype=np.int32), (Hkv, 1))


@pytest.mark.parametrize("D,P,Hq,Hkv,S,g", [
    (128, 64, 8, 2, 4, 8), (64, 16, 4, 1, 8, 8), (128, 32, 8, 1, 5, 8),     # G = 8: two row tiles
    (128, 16, 2, 2, 6, 3), (64, 32, 8, 2, 9, 5), (128, 64, 4, 1, 6, 16)])  # ragged groups, g = 16
def test_tiny_shapes_full(D, P, Hq, Hkv, S, g):
    log(f"[case] fp8qp shape D={D} P={P} Hq={Hq} Hkv={Hkv} S={S} g={g}")
    T = 16 * P
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=D + P + S + g + 1)
    rng = np.random.default_rng(g)
    ids = np.stack([rng.permutation(T) for _ in range(Hkv)]).astype(np.int32)
    O, _, _ = _run(inp, g, ids)
    pairs = [(h, t) for h in range(Hkv) for t in range(T)]
    assert_close_lowp(gpu_rows(O, pairs, Hq // Hkv), model_rows(inp, pairs), f"shape D{D} P{P} g{g}")


def test_rows_independent_of_grouping_and_order():
    # a row's reference maximum and sums follow its own pages only: regrouped (with and without
    # the search's group order), identity and g = 1 outputs are bit-identical
    pw = _pw()
    wl = synth.WORKLOADS["prefill_8k"]
    log("[case] fp8qp prefill_8k: regrouped, ordered, identity and g = 1")
    inp = host_inputs("prefill_8k")
    shp = pw.shape(*wl.shape_tuple())
    dev = pw.to_device(inp)
    ids, order = pw.pw_group_ordered(shp, dev["sel_pages"], wl.W, wl.g)
    O, _, _ = _run(inp, wl.g, ids, dev=dev)
    O_ord, _, _ = _run(inp, wl.g, ids, order=order, dev=dev)
    O_id, _, _ = _run(inp, wl.g, _identity(wl.T, wl.H_kv), dev=dev)
    O_1, _, _ = _run(inp, 1, _identity(wl.T, wl.H_kv), dev=dev)
    for other in (O_ord, O_id, O_1):
        assert torch.equal(O.view(torch.int16), other.view(torch.int16))
    pairs = sample_pairs(wl)
    got = gpu_rows(O, pairs, wl.G)
    assert_close_lowp(got, model_rows(inp, pairs), "prefill_8k")
    # the price of the lower precision, against the method's exact attention
    e = errors(got, oracle_rows(inp, pairs))
    log(f"[accuracy] fp8qp vs exact attention, prefill_8k: max {e['max']:.3e} "
        f"mean {e['mean']:.3e} rel_rms {e['rel_rms']:.3e}")
    assert e["mean"] <= 10 * TOL_MEAN


def test_peaked_and_moving_references():
    # Q x 4 (peaked rows) at 8K, and K scales jumping by up to 2^12 from page to page with V
    # scales over 2^-20 .. 2^20 (the V scale's exponent goes to the MFMA's P scale)
    pw = _pw()
    wl = synth.WORKLOADS["prefill_8k"]
    log("[case] fp8qp prefill_8k peaked")
    inp = host_inputs("prefill_8k", 0, True)
    O, _, _ = _run(inp, wl.g, W=wl.W)
    pairs = sample_pairs(wl, n_random=48)
    got = gpu_rows(O, pairs, wl.G)
    assert_close_lowp(got, model_rows(inp, pairs), "prefill_8k peaked")
    e = errors(got, oracle_rows(inp, pairs))
    log(f"[accuracy] fp8qp vs exact attention, prefill_8k peaked: max {e['max']:.3e} "
        f"mean {e['mean']:.3e} rel_rms {e['rel_rms']:.3e}")

    log("[case] fp8qp moving references, V scales 2^-20 .. 2^20")
    T, P, Hq, Hkv, D, S = 512, 16, 8, 2, 128, 12
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=97)
    sc = inp["scales"].copy()
    N = sc.shape[1]
    rng = np.random.default_rng(5)
    sc[0] = sc[0] * np.exp2(2.0 * (np.arange(N) % 7))[:, None]
    sc[1] = sc[1] * np.exp2(rng.integers(-20, 21, size=sc[1].shape))
    inp = dict(inp, scales=sc.astype(np.float32))
    O, _, _ = _run(inp, 8, W=64)
    pairs = [(h, t) for h in range(Hkv) for t in range(T)]
    got = gpu_rows(O, pairs, Hq // Hkv)
    ref, allow, und = model_rows(inp, pairs)
    # outputs scale with the V scales: compare relative to each row's magnitude
    mag = np.maximum(np.abs(ref).max(axis=2, keepdims=True), 1e-30)
    assert_close_lowp(got / mag, (ref / mag, allow / mag, und), "moving references, wide V scales")


def test_edge_cases_in_selection():
    # empty supports, repeats, out-of-range slots and pages in the causal future
    log("[case] fp8qp selection edge cases")
    T, P, S = 512, 16, 6
    inp = tiny_problem(T=T, Hq=8, Hkv=2, D=128, P=P, S=S, seed=77)
    sel = inp["sel_pages"].copy()
    sel[0, 100] = -1
    sel[1, 7] = [40, 31, -1, 99, -7, 31]
    sel[0, 300] = [18, 18, 0, 0, 31, -1]
    sel[1, 511] = [31, 0, 31, 5, 5, 2]
    inp = dict(inp, sel_pages=sel)
    O, _, _ = _run(inp, 8, W=64)
    pairs = [(h, t) for h in range(2) for t in range(T)]
    assert_close_lowp(gpu_rows(O, pairs, 4), model_rows(inp, pairs), "edge cases")
    o = O.float().cpu().numpy()
    assert np.all(o[100, 0:4] == 0) and np.all(o[7, 4:8] == 0)


def test_edge_cases_in_selection_four_slot_loads():
    # S % 4 == 0 (the union build's 16-byte loads of four slots), two bitset words
    from tests.test_gpu_union_attn import four_slot_edge_selection
    log("[case] fp8qp selection edge cases, S = 8, N = 64")
    inp = four_slot_edge_selection(83)
    O, _, _ = _run(inp, 8, W=64)
    pairs = [(h, t) for h in range(2) for t in range(1024)]
    assert_close_lowp(gpu_rows(O, pairs, 4), model_rows(inp, pairs), "edge cases, S = 8")
    o = O.float().cpu().numpy()
    assert np.all(o[100, 0:4] == 0) and np.all(o[7, 4:8] == 0)


@pytest.mark.parametrize("name,every", [("prefill_64k", 32), ("prefill_64k_70b", 64)])
def test_large_sampled(name, every):
    # the 64K workloads in the benchmark's launch (search with its group order, the re-tiling,
    # the variant in that order; at 70B-like two row tiles per group): every 32nd (64th) window
    # of every head, the first and last two windows and 48 random queries per head
    pw = _pw()
    wl = synth.WORKLOADS[name]
    inp = host_inputs(name)
    pairs = window_sample_pairs(wl, every=every, n_random=48)
    log(f"[case] fp8qp {name}: {len(pairs)} sampled rows")
    shp = pw.shape(*wl.shape_tuple())
    dev = pw.to_device(inp)
    ids, order = pw.pw_group_ordered(shp, dev["sel_pages"], wl.W, wl.g)
    O, _, _ = _run(inp, wl.g, ids, order=order, dev=dev)
    got = gpu_rows(O, pairs, wl.G)
    assert_close_lowp(got, model_rows(inp, pairs), name)
    few = sample_pairs(wl, n_windows=1, n_random=32)
    e = errors(gpu_rows(O, few, wl.G), oracle_rows(inp, few))
    log(f"[accuracy] fp8qp vs exact attention, {name}: max {e['max']:.3e} "
        f"mean {e['mean']:.3e} rel_rms {e['rel_rms']:.3e}")


def test_invalid_arguments():
    pw = _pw()
    inp = tiny_problem(T=64, Hq=4, Hkv=1, D=64, P=16, S=2, seed=1)
    dev = pw.to_device(inp)
    shp = _shape(inp)
    ids = pw.pw_group(shp, dev["sel_pages"], 16, 4)
    ws = pw.pw_tile_kv(shp, dev["k_codes"], dev["v_codes"], dev["scales"])
    with pytest.raises(pw.PWError):
        pw.pw_union_attention_tiled_fp8qp(shp, dev["q_bits"], dev["sel_pages"], ids, 4, ws[:16])
    with pytest.raises(pw.PWError):
        pw.pw_union_attention_tiled_fp8qp(shp, dev["q_bits"], dev["sel_pages"], ids, 0, ws)
