"""pw_dense_union_ref (direct KV-page union) on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from query_union_paged_amd import synth
from tests.gpu_common import assert_close, gpu_rows, host_inputs, log, oracle_rows, sample_pairs
from tests.oracle_helpers import tiny_problem

pytestmark = pytest.mark.gpu


def _run_dense(inp_host):
    from query_union_paged_amd import pageweaver as pw
    dev = pw.to_device(inp_host)
    T, Hq, D = inp_host["q_bits"].shape
    N, Hkv, P, _ = inp_host["k_codes"].shape
    S = inp_host["sel_pages"].shape[2]
    shp = pw.shape(T, Hq, Hkv, D, P, N, S)
    O = pw.pw_dense_union_ref(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"])
    torch.cuda.synchronize()
    return O


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
