"""The binding's documented usage, with torch's own dtypes (bf16 Q, float8_e4m3fn K/V), run as a
user would write it, against the fp64 oracle and the CPU greedy."""
import numpy as np
import pytest
import torch

from oracle.greedy import group_ids
from query_union_paged_amd import synth
from tests.gpu_common import assert_close, gpu_rows, log, oracle_rows

pytestmark = pytest.mark.gpu


def test_documented_usage_with_torch_dtypes():
    from query_union_paged_amd import pageweaver as pw
    wl = synth.WORKLOADS["tiny_1k"]
    inp = synth.make_inputs(wl)
    log(f"[case] usage {wl.name}")
    Q = torch.from_numpy(inp["q_bits"].view(np.int16)).view(torch.bfloat16).cuda()
    K = torch.from_numpy(inp["k_codes"]).view(torch.float8_e4m3fn).cuda()
    V = torch.from_numpy(inp["v_codes"]).view(torch.float8_e4m3fn).cuda()
    scales = torch.from_numpy(inp["scales"]).cuda()
    sel = torch.from_numpy(inp["sel_pages"]).cuda()

    shp = pw.shape_of(Q, K, sel)
    assert (shp.T, shp.H_q, shp.H_kv, shp.D, shp.P, shp.N_pages, shp.S) == wl.shape_tuple()
    ids = pw.pw_group(shp, sel, W=wl.W, g=wl.g)
    O = pw.pw_union_attention(shp, Q, K, V, scales, sel, ids, wl.g)

    ids2, order = pw.pw_group_ordered(shp, sel, wl.W, wl.g)
    ws = pw.pw_tile_kv(shp, K, V, scales)
    O2 = pw.pw_union_attention_tiled(shp, Q, sel, ids2, wl.g, ws, group_order=order)
    torch.cuda.synchronize()

    assert O.dtype == torch.bfloat16 and tuple(O.shape) == (wl.T, wl.H_q, wl.D)
    ref_ids = group_ids(inp["sel_pages"], wl.N, wl.W, wl.g)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.array_equal(ids2.cpu().numpy(), ref_ids)
    # the ordered call computes every row exactly as the plain one does
    assert torch.equal(O.view(torch.int16), O2.view(torch.int16))
    pairs = [(h, t) for h in range(wl.H_kv) for t in range(wl.T)]
    G = wl.H_q // wl.H_kv
    assert_close(gpu_rows(O, pairs, G), oracle_rows(inp, pairs), "documented usage, tiny")
