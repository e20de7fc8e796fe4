"""pw_union_attention on the GPU against the fp64 oracle (element by element)."""
import numpy as np
import pytest
import torch

from query_union_paged_amd import synth
from tests.gpu_common import (assert_close, gpu_rows, host_inputs, log, oracle_rows,
                              sample_pairs, window_sample_pairs)
from tests.oracle_helpers import tiny_problem

pytestmark = pytest.mark.gpu


def _pw():
    from query_union_paged_amd import pageweaver
    return pageweaver


def _run(inp_host, g, ids_mode="regroup", W=None):
    """Upload, build IDs (GPU search, identity or given), run the union kernel."""
    pw = _pw()
    dev = pw.to_device(inp_host)
    T, Hq, D = inp_host["q_bits"].shape
    N, Hkv, P, _ = inp_host["k_codes"].shape
    S = inp_host["sel_pages"].shape[2]
    shp = pw.shape(T, Hq, Hkv, D, P, N, S)
    if isinstance(ids_mode, np.ndarray):
        ids = torch.from_numpy(ids_mode).cuda()
    elif ids_mode == "regroup":
        ids = pw.pw_group(shp, dev["sel_pages"], W, g)
    else:
        ids = torch.arange(T, dtype=torch.int32, device="cuda").repeat(Hkv, 1).contiguous()
    O = pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, g)
    torch.cuda.synchronize()
    return O, ids


def _all_pairs(Hkv, T):
    return [(h, t) for h in range(Hkv) for t in range(T)]


@pytest.mark.parametrize("variant,peaked", [(0, False), (1, False), (2, False), (0, True)])
@pytest.mark.parametrize("arm", ["regroup", "identity", "g1"])
def test_tiny_full(variant, peaked, arm):
    wl = synth.WORKLOADS["tiny_1k"]
    log(f"[case] union tiny_1k v{variant} peaked={peaked} arm={arm}")
    inp = host_inputs("tiny_1k", variant, peaked)
    g = 1 if arm == "g1" else wl.g
    O, _ = _run(inp, g, "identity" if arm == "identity" else "regroup", wl.W)
    pairs = _all_pairs(wl.H_kv, wl.T)
    assert_close(gpu_rows(O, pairs, wl.G), oracle_rows(inp, pairs), f"tiny v{variant} {arm}")


def test_8k_full_and_arm_identity():
    wl = synth.WORKLOADS["prefill_8k"]
    log("[case] union prefill_8k full")
    inp = host_inputs("prefill_8k")
    O_r, ids = _run(inp, wl.g, "regroup", wl.W)
    pairs = _all_pairs(wl.H_kv, wl.T)
    ref = oracle_rows(inp, pairs)
    assert_close(gpu_rows(O_r, pairs, wl.G), ref, "8k regroup")
    O_i, _ = _run(inp, wl.g, "identity")
    # a row's result does not depend on the group it sits in
    same = (O_r.float() == O_i.float()).float().mean().item()
    log(f"[parity] 8k regroup vs identity: fraction of equal elements {same:.6f}")
    assert same == 1.0
    O_1, _ = _run(inp, 1, "identity")
    assert (O_1.float() == O_r.float()).all()
    # run-to-run determinism
    O_r2, ids2 = _run(inp, wl.g, "regroup", wl.W)
    assert torch.equal(ids, ids2) and torch.equal(O_r.view(torch.int16), O_r2.view(torch.int16))


def test_8k_peaked_sampled():
    wl = synth.WORKLOADS["prefill_8k"]
    log("[case] union prefill_8k peaked")
    inp = host_inputs("prefill_8k", 0, True)
    O, _ = _run(inp, wl.g, "regroup", wl.W)
    pairs = sample_pairs(wl)
    assert_close(gpu_rows(O, pairs, wl.G), oracle_rows(inp, pairs), "8k peaked")


@pytest.mark.parametrize("D,P,Hq,Hkv,S,g", [
    (64, 16, 4, 1, 8, 8), (64, 32, 8, 2, 5, 8), (128, 64, 8, 1, 4, 8),   # G = 8: two row tiles
    (128, 16, 2, 2, 6, 8), (64, 64, 16, 2, 3, 4), (128, 32, 4, 2, 7, 3),  # g = 3: ragged last group
    (128, 64, 1, 1, 5, 8), (64, 16, 8, 4, 9, 5), (128, 64, 32, 1, 3, 2),
    (128, 64, 4, 1, 6, 16), (64, 16, 8, 2, 9, 16), (128, 32, 2, 2, 5, 13),   # g up to 16
    (128, 16, 4, 1, 64, 16)])                                               # g * S = 1024
def test_shapes_and_group_sizes(D, P, Hq, Hkv, S, g):
    log(f"[case] union shape D={D} P={P} Hq={Hq} Hkv={Hkv} S={S} g={g}")
    T = 16 * P
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=D + P + S + g)
    rng = np.random.default_rng(g)
    ids = np.stack([rng.permutation(T) for _ in range(Hkv)]).astype(np.int32)
    O, _ = _run(inp, g, ids)
    pairs = _all_pairs(Hkv, T)
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), f"shape D{D} P{P} g{g}")


def test_edge_cases_in_selection():
    # empty supports, repeats, out-of-range slots and pages in the causal future
    log("[case] union selection edge cases")
    T, P, S = 512, 16, 6
    inp = tiny_problem(T=T, Hq=8, Hkv=2, D=128, P=P, S=S, seed=77)
    sel = inp["sel_pages"].copy()
    sel[0, 100] = -1                         # empty support -> O = 0
    sel[1, 7] = [40, 31, -1, 99, -7, 31]     # only future / out-of-range pages -> O = 0
    sel[0, 300] = [18, 18, 0, 0, 31, -1]     # repeats and one future page
    sel[1, 511] = [31, 0, 31, 5, 5, 2]
    inp = dict(inp, sel_pages=sel)
    O, _ = _run(inp, 8, "regroup", 64)
    pairs = _all_pairs(2, T)
    got = gpu_rows(O, pairs, 4)
    ref = oracle_rows(inp, pairs)
    assert_close(got, ref, "edge cases")
    o = O.float().cpu().numpy()
    assert np.all(o[100, 0:4] == 0) and np.all(o[7, 4:8] == 0)


def four_slot_edge_selection(seed):
    """T = 1024, P = 16 (N = 64 pages: two bitset words), S = 8 (each member row is two 16-byte
    loads of four slots): invalid slots between valid ones, repeats, out-of-range and future
    pages, unsorted rows alternating between the two words, a row of one page."""
    T, P, S = 1024, 16, 8
    inp = tiny_problem(T=T, Hq=8, Hkv=2, D=128, P=P, S=S, seed=seed)
    sel = inp["sel_pages"].copy()
    sel[0, 100] = -1                                    # empty support -> O = 0
    sel[1, 7] = [40, 63, -1, 99, -7, 33, 64, 2]         # only future / out-of-range pages -> O = 0
    sel[0, 300] = [18, 18, 0, 0, 37, -1, 5, 5]          # repeats around an invalid slot
    sel[1, 511] = [33, 2, 40, 1, 63, 32, 0, 31]         # unsorted, alternating words
    sel[0, 900] = [49, 50, -1, 51, 49, 99, 52, 50]      # a same-word run cut by invalid slots
    sel[1, 1000] = 56                                   # one page in every slot
    sel[0, 40:48] = sel[0, 40:48][:, ::-1]              # descending rows
    return dict(inp, sel_pages=sel)


def test_edge_cases_in_selection_four_slot_loads():
    # S % 4 == 0: the union build reads four slots of a member with one 16-byte load and ORs
    # the entries of one bitset word with one LDS atomic
    log("[case] union selection edge cases, S = 8, N = 64")
    inp = four_slot_edge_selection(81)
    O, _ = _run(inp, 8, "regroup", 64)
    pairs = _all_pairs(2, 1024)
    assert_close(gpu_rows(O, pairs, 4), oracle_rows(inp, pairs), "edge cases, S = 8")
    o = O.float().cpu().numpy()
    assert np.all(o[100, 0:4] == 0) and np.all(o[7, 4:8] == 0)


@pytest.mark.parametrize("name,arms", [("prefill_32k", ["regroup", "identity"]),
                                       ("prefill_64k", ["regroup", "identity", "g1"]),
                                       ("prefill_64k_70b", ["regroup", "identity"])])
def test_large_sampled(name, arms):
    # every 16th window of every head, the first and last two windows, 96 random queries per head
    wl = synth.WORKLOADS[name]
    inp = host_inputs(name)
    pairs = window_sample_pairs(wl)
    ref = oracle_rows(inp, pairs)
    log(f"[case] union {name}: {len(pairs)} sampled rows")
    for arm in arms:
        log(f"[case] union {name} arm={arm}")
        g = 1 if arm == "g1" else wl.g
        O, ids = _run(inp, g, "identity" if arm == "identity" else "regroup", wl.W)
        assert_close(gpu_rows(O, pairs, wl.G), ref, f"{name} {arm}")
        if arm == "regroup":
            # the same call with the search's size order: bit-identical rows
            pw = _pw()
            dev = pw.to_device(inp)
            shp = pw.shape(*wl.shape_tuple())
            ids_o, order = pw.pw_group_ordered(shp, dev["sel_pages"], wl.W, wl.g)
            ws = pw.pw_tile_kv(shp, dev["k_codes"], dev["v_codes"], dev["scales"])
            O_o = pw.pw_union_attention_tiled(shp, dev["q_bits"], dev["sel_pages"], ids_o, wl.g,
                                              ws, group_order=order)
            torch.cuda.synchronize()
            assert torch.equal(ids_o, ids)
            assert torch.equal(O_o.view(torch.int16), O.view(torch.int16))
            del dev, ws, O_o
        del O
        torch.cuda.empty_cache()


def test_invalid_arguments_raise():
    pw = _pw()
    inp = tiny_problem(T=64, Hq=4, Hkv=1, D=64, P=16, S=2, seed=1)
    dev = pw.to_device(inp)
    shp = pw.shape(64, 4, 1, 64, 16, 4, 2)
    ids = torch.arange(64, dtype=torch.int32, device="cuda")[None].contiguous()
    with pytest.raises(pw.PWError) as e:
        pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, 17)
    assert e.value.status == pw.PW_ERR_UNSUPPORTED
    bad = pw.shape(64, 4, 1, 64, 16, 5, 2)
    with pytest.raises((pw.PWError, ValueError)):
        pw.pw_union_attention(bad, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, 8)


def test_largest_page_count():
    # N_pages = 32768 (the supported maximum) at P = 16: T = 524288 queries, identity groups;
    # the largest union list and page bitset; page offsets of the tiled copy reach
    # 32768 * 64 * 64 = 2^27 bytes (the 2^31 limit of the offsets is checked on the host,
    # test_abi.py)
    T, P, Hq, Hkv, D, S, g = 524288, 16, 4, 1, 64, 4, 8
    N = T // P
    log(f"[case] union largest N={N} T={T}")
    rng = np.random.default_rng(5)
    gen = torch.Generator().manual_seed(5)
    t = np.arange(T)
    own = t // P
    sel = np.stack([np.zeros(T, np.int64), own, own - 1, (rng.random(T) * (own + 1)).astype(np.int64)],
                   axis=1)
    sel = np.where(sel < 0, -1, sel).astype(np.int32)[None]            # [1][T][4], repeats allowed
    inp = {
        "q_bits": torch.randn((T, Hq, D), generator=gen).to(torch.bfloat16)
                       .view(torch.int16).numpy().view(np.uint16),
        "k_codes": torch.randn((N, Hkv, P, D), generator=gen).to(torch.float8_e4m3fn)
                        .view(torch.uint8).numpy(),
        "v_codes": torch.randn((N, Hkv, P, D), generator=gen).to(torch.float8_e4m3fn)
                        .view(torch.uint8).numpy(),
        "scales": rng.uniform(0.05, 1.0, size=(2, N, Hkv)).astype(np.float32),
        "sel_pages": sel,
    }
    O, _ = _run(inp, g, "identity")
    pick = np.concatenate([np.arange(64), np.arange(T - 64, T),
                           rng.choice(T, size=128, replace=False)])
    pairs = sorted({(0, int(x)) for x in pick})
    assert_close(gpu_rows(O, pairs, Hq), oracle_rows(inp, pairs), "largest N")


def test_side_streams_and_concurrent_calls():
    # every call runs on the stream it is given: two side streams with their own workspaces,
    # enqueued back to back, reproduce the default-stream results bit for bit
    pw = _pw()
    wl = synth.WORKLOADS["prefill_8k"]
    log("[case] side streams")
    inp = host_inputs("prefill_8k")
    dev = pw.to_device(inp)
    shp = pw.shape(*wl.shape_tuple())
    ids = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    ref = pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                                dev["sel_pages"], ids, wl.g)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, idss = [], []
    for s in streams:
        with torch.cuda.stream(s):
            i_s = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g, stream=s)
            o_s = pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"],
                                        dev["scales"], dev["sel_pages"], i_s, wl.g, stream=s)
            idss.append(i_s)
            outs.append(o_s)
    torch.cuda.synchronize()
    for i_s, o_s in zip(idss, outs):
        assert torch.equal(i_s, ids)
        assert torch.equal(o_s.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("chunk", [1, 2, 4])
def test_head_pipeline_matches_the_plain_call(chunk):
    # search of later KV heads on a second stream while earlier heads attend: same IDs and
    # the same output bits as pw_group + pw_union_attention on one stream
    pw = _pw()
    wl = synth.WORKLOADS["prefill_8k"]
    log(f"[case] head pipeline prefill_8k chunk={chunk}")
    dev = pw.to_device(host_inputs("prefill_8k"))
    shp = pw.shape(*wl.shape_tuple())
    ws = torch.empty(pw.pw_union_attention_workspace_bytes(shp, wl.g), dtype=torch.uint8,
                     device="cuda")
    ids_ref = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    O_ref = pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"],
                                  dev["scales"], dev["sel_pages"], ids_ref, wl.g, workspace=ws)
    run = pw.HeadPipeline(shp, chunk)
    ids = torch.full_like(ids_ref, -7)
    O = torch.zeros_like(O_ref)
    for _ in range(2):                          # twice: events and streams are reused
        run(dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"], dev["sel_pages"],
            wl.W, wl.g, ids, O, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_ref)
    assert torch.equal(O.view(torch.int16), O_ref.view(torch.int16))


def test_head_range_writes_only_its_heads():
    pw = _pw()
    log("[case] pw_union_attention_heads (1, 2) of 4 KV heads")
    T, Hq, Hkv, D, P, S = 256, 8, 4, 64, 16, 6
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=5)
    dev = pw.to_device(inp)
    shp = pw.shape(T, Hq, Hkv, D, P, T // P, S)
    ids = torch.arange(T, dtype=torch.int32, device="cuda").repeat(Hkv, 1).contiguous()
    O = torch.full((T, Hq, D), 3.0, dtype=torch.bfloat16, device="cuda")
    pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                          dev["sel_pages"], ids, 8, O=O, heads=(1, 2))
    torch.cuda.synchronize()
    pairs = [(h, t) for h in (1, 2) for t in range(T)]
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), "head range")
    G = Hq // Hkv
    untouched = torch.cat([O[:, :G], O[:, 3 * G:]], dim=1).float()
    assert bool((untouched == 3.0).all())
    with pytest.raises(pw.PWError) as e:
        pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, 8, O=O, heads=(2, 3))
    assert e.value.status == pw.PW_ERR_DIMS


def test_extreme_magnitudes():
    # Q rows scaled by 2^-40 .. 2^4 (the per-row power-of-two split must keep them exact) and
    # K scales from 1e-4 to 10 (very flat to very peaked softmax rows, logits up to ~1e4 in
    # log2 units; the documented range is |logit| < 2^20), V scales unchanged
    log("[case] union extreme Q magnitudes and K scales")
    T, P, Hq, Hkv, D, S = 256, 16, 8, 2, 128, 7
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=91)
    q = torch.from_numpy(inp["q_bits"].view(np.int16)).view(torch.bfloat16).float()
    e = torch.from_numpy(np.random.default_rng(1).integers(-40, 5, size=(T, Hq, 1))).float()
    q = (q * torch.exp2(e)).to(torch.bfloat16)
    sc = inp["scales"].copy()
    sc[0] = np.exp(np.random.default_rng(2).uniform(np.log(1e-4), np.log(10.0), size=sc[0].shape))
    inp = dict(inp, q_bits=q.view(torch.int16).numpy().view(np.uint16), scales=sc.astype(np.float32))
    O, _ = _run(inp, 8, "regroup", 32)
    pairs = _all_pairs(Hkv, T)
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), "extreme magnitudes")


def test_moving_reference_maximum():
    # K scales that jump by 2^0 .. 2^12 from page to page: the row maxima of some pages pass the
    # running reference by more than the lazy threshold (rescales), those of the pages after a
    # jump cannot (the norm bound lets the wave skip its max pass); all within tolerance, and
    # regrouped, identity and g = 1 rows stay bit-identical
    log("[case] union moving reference maximum")
    T, P, Hq, Hkv, D, S = 512, 16, 8, 2, 128, 12
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=93)
    sc = inp["scales"].copy()
    N = sc.shape[1]
    sc[0] = sc[0] * np.exp2(2.0 * (np.arange(N) % 7))[:, None]
    inp = dict(inp, scales=sc.astype(np.float32))
    O, _ = _run(inp, 8, "regroup", 64)
    pairs = _all_pairs(Hkv, T)
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), "moving reference")
    O_id, _ = _run(inp, 8, "identity")
    O_1, _ = _run(inp, 1, "identity")
    assert torch.equal(O.view(torch.int16), O_id.view(torch.int16))
    assert torch.equal(O.view(torch.int16), O_1.view(torch.int16))


def test_tight_score_bound():
    # every Q row is a power-of-two multiple of one key of a page it selected, so that page's
    # best score equals |q| * max |k| (the norm bound is tight, up to rounding); the rows reach
    # logits of several tens, so the bound decides between skipping and computing row maxima
    # right at the lazy threshold
    log("[case] union tight score bound")
    T, P, Hq, Hkv, D, S = 512, 16, 4, 1, 128, 8
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=95)
    rng = np.random.default_rng(7)
    kdec = torch.from_numpy(inp["k_codes"]).view(torch.float8_e4m3fn).float().numpy()
    sel = inp["sel_pages"]
    q = np.zeros((T, Hq, D), np.float32)
    for t in range(T):
        pages = sel[0, t][(sel[0, t] >= 0) & (sel[0, t] * P <= t)]
        for j in range(Hq):
            u = int(rng.choice(pages))
            c = int(rng.integers(0, min(P, t - u * P + 1)))
            q[t, j] = kdec[u, 0, c] * 2.0 ** int(rng.integers(-2, 3))
    qb = torch.from_numpy(q).to(torch.bfloat16)
    assert torch.equal(qb.float(), torch.from_numpy(q))          # exact in bf16
    inp = dict(inp, q_bits=qb.view(torch.int16).numpy().view(np.uint16))
    O, _ = _run(inp, 8, "regroup", 64)
    pairs = _all_pairs(Hkv, T)
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), "tight score bound")
    O_id, _ = _run(inp, 8, "identity")
    assert torch.equal(O.view(torch.int16), O_id.view(torch.int16))


@pytest.mark.parametrize("T,P,g,W", [(16, 16, 16, 16), (16, 16, 8, 16), (32, 16, 1, 32), (64, 64, 4, 64)])
def test_minimal_shapes(T, P, g, W):
    # one or two pages, a window equal to the sequence, groups of one or of the whole sequence
    log(f"[case] union minimal T={T} P={P} g={g} W={W}")
    inp = tiny_problem(T=T, Hq=4, Hkv=1, D=64, P=P, S=2, seed=T + g)
    O, ids = _run(inp, g, "regroup", W)
    assert sorted(ids.cpu().numpy()[0].tolist()) == list(range(T))
    pairs = _all_pairs(1, T)
    assert_close(gpu_rows(O, pairs, 4), oracle_rows(inp, pairs), f"minimal T={T} g={g}")


@pytest.mark.parametrize("W,g", [(512, 8), (1024, 16)])
def test_wide_window_pipeline(W, g):
    # a wide search window (several waves per window) feeding the attention
    wl = synth.WORKLOADS["prefill_8k"]
    log(f"[case] union prefill_8k regrouped with W={W} g={g}")
    inp = host_inputs("prefill_8k")
    O, ids = _run(inp, g, "regroup", W)
    rows = sample_pairs(wl)
    assert_close(gpu_rows(O, rows, wl.G), oracle_rows(inp, rows), f"wide window W={W} g={g}")


def test_disjoint_head_ranges_share_a_workspace_concurrently():
    # two streams, KV heads [0, 4) and [4, 8), one workspace: the same bits as one full call
    pw = _pw()
    wl = synth.WORKLOADS["prefill_8k"]
    log("[case] pw_union_attention_heads on two streams with one workspace")
    dev = pw.to_device(host_inputs("prefill_8k"))
    shp = pw.shape(*wl.shape_tuple())
    ws = torch.empty(pw.pw_union_attention_workspace_bytes(shp, wl.g), dtype=torch.uint8,
                     device="cuda")
    ids = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    args = (shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"], dev["sel_pages"],
            ids, wl.g)
    O_ref = pw.pw_union_attention(*args, workspace=ws)
    torch.cuda.synchronize()
    ws.zero_()
    O = torch.zeros_like(O_ref)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        pw.pw_union_attention(*args, O=O, workspace=ws, stream=s1, heads=(0, 4))
        pw.pw_union_attention(*args, O=O, workspace=ws, stream=s2, heads=(4, 4))
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O_ref.view(torch.int16))


@pytest.mark.parametrize("name", ["prefill_8k", "shape_g8", "ragged"])
def test_group_order_leaves_every_row_unchanged(name):
    # pw_union_attention_tiled_ordered: the search's size order, a random permutation and the
    # plain order give bit-identical outputs; an order entry outside the group range runs no
    # group (its rows keep their previous contents)
    pw = _pw()
    log(f"[case] ordered attention {name}")
    if name == "prefill_8k":
        wl = synth.WORKLOADS[name]
        inp, g, W = host_inputs(name), wl.g, wl.W
    elif name == "shape_g8":                # G = 8: two 32-row tiles per group
        inp, g, W = tiny_problem(T=2048, P=32, Hq=16, Hkv=2, D=128, S=10, seed=11), 8, 64
    else:                                   # T = 1008, g = 5: the last group has 3 members
        inp, g, W = tiny_problem(T=1008, P=16, Hq=8, Hkv=2, D=64, S=6, seed=5), 5, 35
    dev = pw.to_device(inp)
    T, Hq, D = inp["q_bits"].shape
    N, Hkv, P, _ = inp["k_codes"].shape
    S = inp["sel_pages"].shape[2]
    shp = pw.shape(T, Hq, Hkv, D, P, N, S)
    ids, order = pw.pw_group_ordered(shp, dev["sel_pages"], W, g)
    ws = pw.pw_tile_kv(shp, dev["k_codes"], dev["v_codes"], dev["scales"])
    plain = pw.pw_union_attention_tiled(shp, dev["q_bits"], dev["sel_pages"], ids, g, ws)
    sized = pw.pw_union_attention_tiled(shp, dev["q_bits"], dev["sel_pages"], ids, g, ws,
                                        group_order=order)
    ng = order.shape[1]
    perm = torch.stack([torch.randperm(ng, generator=torch.Generator().manual_seed(h))
                        for h in range(Hkv)]).to(torch.int32).cuda()
    shuffled = pw.pw_union_attention_tiled(shp, dev["q_bits"], dev["sel_pages"], ids, g, ws,
                                           group_order=perm)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), sized.view(torch.int16))
    assert torch.equal(plain.view(torch.int16), shuffled.view(torch.int16))
    # group 3 of head 0 is replaced by an out-of-range entry: its rows stay as they were
    bad = order.clone()
    pos = int((bad[0] == 3).nonzero()[0, 0])
    bad[0, pos] = ng
    O = torch.full_like(plain, 7.0)
    pw.pw_union_attention_tiled(shp, dev["q_bits"], dev["sel_pages"], ids, g, ws, O=O,
                                group_order=bad)
    torch.cuda.synchronize()
    G = Hq // Hkv
    miss = ids[0, 3 * g:4 * g].long().cpu()
    heads0 = slice(0, G)
    assert torch.all(O[miss][:, heads0] == 7.0)
    keep = torch.ones(T, dtype=torch.bool)
    keep[miss] = False
    assert torch.equal(O[keep].view(torch.int16), plain[keep].view(torch.int16))
    assert torch.equal(O[miss][:, G:].view(torch.int16), plain[miss][:, G:].view(torch.int16))
