"""pw_dense_union_ref / pw_dense_union_paired (direct KV-page union) and pw_page_pairs on the
GPU against the fp64 oracle: outputs within the attention tolerance, affinity pairs bit-exact."""
import numpy as np
import pytest
import torch

from query_union_paged_amd import synth
from tests.gpu_common import assert_close, gpu_rows, host_inputs, log, oracle_rows, sample_pairs
from tests.oracle_helpers import tiny_problem

pytestmark = pytest.mark.gpu


def _run_dense(inp_host, affinity=False):
    from query_union_paged_amd import pageweaver as pw
    dev = pw.to_device(inp_host)
    T, Hq, D = inp_host["q_bits"].shape
    N, Hkv, P, _ = inp_host["k_codes"].shape
    S = inp_host["sel_pages"].shape[2]
    shp = pw.shape(T, Hq, Hkv, D, P, N, S)
    pairs = pw.pw_page_pairs(shp, dev["sel_pages"]) if affinity else None
    O = pw.pw_dense_union_ref(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], pairs=pairs)
    torch.cuda.synchronize()
    return (O, pairs.cpu().numpy()) if affinity else O


def _oracle_pairs(sel, N, heads):
    from oracle.dense_union import affinity_pairs
    return {h: affinity_pairs(sel[h], N) for h in heads}


def _assert_pairs(got, ref, N):
    for h, pr in ref.items():
        want = np.full((N, 2), -1, dtype=np.int32)
        want[:len(pr)] = np.array(pr, dtype=np.int32)
        assert np.array_equal(got[h], want), f"head {h}: {(got[h] != want).any(axis=1).sum()} rows differ"


@pytest.mark.parametrize("variant,peaked", [(0, False), (1, False), (0, True)])
def test_dense_tiny_full(variant, peaked):
    wl = synth.WORKLOADS["tiny_1k"]
    log(f"[case] dense tiny_1k v{variant} peaked={peaked}")
    inp = host_inputs("tiny_1k", variant, peaked)
    O = _run_dense(inp)
    pairs = [(h, t) for h in range(wl.H_kv) for t in range(wl.T)]
    assert_close(gpu_rows(O, pairs, wl.G), oracle_rows(inp, pairs), f"dense tiny v{variant}")


@pytest.mark.parametrize("name", ["prefill_8k", "prefill_64k_70b"])
def test_dense_sampled(name):
    wl = synth.WORKLOADS[name]
    log(f"[case] dense {name}")
    inp = host_inputs(name)
    O = _run_dense(inp)
    pairs = sample_pairs(wl)
    assert_close(gpu_rows(O, pairs, wl.G), oracle_rows(inp, pairs), f"dense {name}")


@pytest.mark.parametrize("D,P,Hq,Hkv,S", [(64, 16, 4, 1, 8), (128, 32, 8, 2, 5), (128, 64, 8, 1, 7),
                                          (64, 64, 2, 2, 3)])
def test_dense_shapes(D, P, Hq, Hkv, S):
    log(f"[case] dense shape D={D} P={P} Hq={Hq} Hkv={Hkv} S={S}")
    T = 16 * P
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=D * P + S)
    sel = inp["sel_pages"].copy()
    sel[0, T // 2] = -1                       # an empty support -> O = 0
    sel[-1, 3, 0] = 15                        # a page in the causal future
    inp = dict(inp, sel_pages=sel)
    O = _run_dense(inp)
    pairs = [(h, t) for h in range(Hkv) for t in range(T)]
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), f"dense shape D{D} P{P}")


@pytest.mark.parametrize("variant,peaked", [(0, False), (1, True)])
def test_dense_affinity_tiny_full(variant, peaked):
    wl = synth.WORKLOADS["tiny_1k"]
    log(f"[case] dense affinity tiny_1k v{variant} peaked={peaked}")
    inp = host_inputs("tiny_1k", variant, peaked)
    O, got = _run_dense(inp, affinity=True)
    _assert_pairs(got, _oracle_pairs(inp["sel_pages"], wl.N, range(wl.H_kv)), wl.N)
    pairs = [(h, t) for h in range(wl.H_kv) for t in range(wl.T)]
    assert_close(gpu_rows(O, pairs, wl.G), oracle_rows(inp, pairs), f"dense affinity tiny v{variant}")


@pytest.mark.parametrize("name", ["prefill_8k", "prefill_64k_70b"])
def test_dense_affinity_sampled(name):
    wl = synth.WORKLOADS[name]
    log(f"[case] dense affinity {name}")
    inp = host_inputs(name)
    O, got = _run_dense(inp, affinity=True)
    heads = range(wl.H_kv) if wl.T <= 8192 else [0, wl.H_kv - 1]
    _assert_pairs(got, _oracle_pairs(inp["sel_pages"], wl.N, heads), wl.N)
    rows = sample_pairs(wl)
    assert_close(gpu_rows(O, rows, wl.G), oracle_rows(inp, rows), f"dense affinity {name}")


@pytest.mark.parametrize("T,P,S,seed", [(1024, 16, 6, 0), (2048, 16, 9, 1), (1000, 8, 4, 2),
                                        (4096, 2, 5, 3)])
def test_page_pairs_random(T, P, S, seed):
    # random and clustered selections (many equal counts), N up to 2048 pages, ragged T
    from query_union_paged_amd import pageweaver as pw
    log(f"[case] pw_page_pairs T={T} P={P} S={S}")
    rng = np.random.default_rng(seed)
    N = -(-T // P)
    T = N * P
    sel = rng.integers(-2, N + 2, size=(2, T, S)).astype(np.int32)
    sel[:, ::3] %= 7
    sel[1, 5::11] = sel[1, 5]                   # repeated rows
    shp = pw.shape(T, 2, 2, 64, P, N, S)
    got = pw.pw_page_pairs(shp, torch.from_numpy(sel).cuda())
    again = pw.pw_page_pairs(shp, torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.array_equal(got, again.cpu().numpy())
    _assert_pairs(got, _oracle_pairs(sel, N, range(2)), N)


@pytest.mark.parametrize("D,P,Hq,Hkv,S", [(64, 16, 4, 1, 8), (128, 32, 8, 2, 5)])
def test_dense_affinity_shapes(D, P, Hq, Hkv, S):
    log(f"[case] dense affinity shape D={D} P={P} Hq={Hq} Hkv={Hkv} S={S}")
    T = 32 * P
    inp = tiny_problem(T=T, Hq=Hq, Hkv=Hkv, D=D, P=P, S=S, seed=D + P + S)
    O, got = _run_dense(inp, affinity=True)
    _assert_pairs(got, _oracle_pairs(inp["sel_pages"], T // P, range(Hkv)), T // P)
    pairs = [(h, t) for h in range(Hkv) for t in range(T)]
    assert_close(gpu_rows(O, pairs, Hq // Hkv), oracle_rows(inp, pairs), f"dense affinity D{D} P{P}")
