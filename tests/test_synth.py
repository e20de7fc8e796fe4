"""Invariants of the seeded generator (CPU only)."""
import numpy as np
import pytest

from query_union_paged_amd import synth
from oracle.fp8 import decode_e4m3fn


@pytest.mark.parametrize("name", ["tiny_1k", "prefill_8k"])
def test_selection_invariants(name):
    wl = synth.WORKLOADS[name]
    sel = synth.make_selection(wl)
    assert sel.shape == (wl.H_kv, wl.T, wl.S) and sel.dtype == np.int32
    t = np.arange(wl.T)
    p = t // wl.P
    n = np.minimum(wl.S, p + 1)
    valid = sel >= 0
    assert np.array_equal(valid.sum(axis=2), np.broadcast_to(n, valid.shape[:2]))
    # valid entries first, ascending and unique, then -1 padding
    assert np.all(valid[:, :, :-1] | ~valid[:, :, 1:])
    d = np.diff(sel, axis=2)
    assert np.all((d > 0) | ~valid[:, :, 1:])
    assert np.all(np.where(valid, sel <= p[None, :, None], True))           # causal
    assert np.all(sel[:, :, 0] == 0)                                        # sink
    assert np.all((sel == p[None, :, None]).any(axis=2))                    # own page
    if wl.n_local == 2:
        q = t[p >= 1]
        assert np.all((sel[:, q] == (p[q] - 1)[None, :, None]).any(axis=2))


def test_useful_flops_closed_form():
    for name in ["tiny_1k", "prefill_8k"]:
        wl = synth.WORKLOADS[name]
        sel = synth.make_selection(wl)
        t = np.arange(wl.T)
        p = t // wl.P
        closed = wl.H_kv * wl.G * 4 * wl.D * np.sum((np.minimum(wl.S, p + 1) - 1) * wl.P + (t % wl.P) + 1)
        assert synth.useful_flops(sel, wl) == float(closed)


def test_seeded_and_parallel_reproducible():
    wl = synth.WORKLOADS["prefill_8k"]
    a = synth.make_selection(wl)
    b = synth.make_selection(wl, workers=4)
    c = synth.make_selection(wl, variant=1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_alternating_structure():
    # adjacent queries draw from different community sets: their overlap is small
    wl = synth.WORKLOADS["prefill_8k"]
    sel = synth.make_selection(wl)
    h, t = 0, np.arange(4096, 4160)
    sets = [set(sel[h, x].tolist()) - {-1} for x in t]
    adj = np.mean([len(sets[i] & sets[i + 1]) for i in range(0, 63, 2)])
    same = np.mean([len(sets[i] & sets[i + 2]) for i in range(0, 62, 2)])
    assert same > adj + 5


def test_kv_quantisation():
    wl = synth.WORKLOADS["tiny_1k"]
    d = synth.make_qkv(wl)
    kc, vc, sc = d["k_codes"], d["v_codes"], d["scales"]
    assert kc.shape == (wl.N, wl.H_kv, wl.P, wl.D) and vc.shape == (wl.N, wl.H_kv, wl.P, wl.D)
    for codes in (kc, vc):
        vals = decode_e4m3fn(codes)
        assert not np.isnan(vals).any()
        assert np.all(np.abs(vals).reshape(wl.N, wl.H_kv, -1).max(axis=2) == 448.0)
    assert sc.dtype == np.float32 and np.all(sc > 0)
    # dequantised values approximate the bf16 source within e4m3 rounding (2^-4 relative)
    import torch
    gen = torch.Generator().manual_seed(wl.seed_for(0))
    torch.randn((wl.T, wl.H_q, wl.D), generator=gen)
    k = torch.randn((wl.N, wl.H_kv, wl.P, wl.D), generator=gen).to(torch.bfloat16).double().numpy()
    khat = decode_e4m3fn(kc) * sc[0][:, :, None, None]
    err = np.abs(khat - k)
    assert np.all(err <= np.abs(k) * 2 ** -4 + sc[0].max() * 2 ** -9 + 1e-12)


def test_peaked_variant_scales_q():
    wl = synth.WORKLOADS["tiny_1k"]
    a = synth.make_qkv(wl)["q_bits"]
    b = synth.make_qkv(wl, peaked=True)["q_bits"]
    from oracle.fp8 import decode_bf16
    np.testing.assert_array_equal(decode_bf16(b), 4 * decode_bf16(a))
