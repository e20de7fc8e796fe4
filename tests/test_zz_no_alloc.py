"""pw_union_attention_noalloc against pw_union_attention (GPU, through the C ABI).

Two calls in a row on one device, the second on a smaller problem: each must
give exactly the output of the workspace entry point (same kernels, same
inputs), so the shared scratch holds nothing from the previous call that
matters.
"""
import numpy as np
import pytest
import torch

from query_union_paged_amd import synth
from gpu_common import host_inputs, log

pytestmark = pytest.mark.gpu


def _both(name):
    from query_union_paged_amd import pageweaver as pw
    wl = synth.WORKLOADS[name]
    inp = host_inputs(name)
    dev = pw.to_device(inp)
    shp = pw.shape(*wl.shape_tuple())
    ids = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    args = (shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"], dev["sel_pages"],
            ids, wl.g)
    O_ws = pw.pw_union_attention(*args)
    O_na = torch.full_like(O_ws, float("nan"))
    pw.pw_union_attention_noalloc(*args, O=O_na)
    torch.cuda.synchronize()
    return O_ws, O_na


def test_noalloc_matches_workspace_call_twice():
    for name in ("prefill_8k", "tiny_1k"):          # the second call is the smaller problem
        log(f"[case] pw_union_attention_noalloc vs pw_union_attention, {name}")
        O_ws, O_na = _both(name)
        assert torch.isfinite(O_na.float()).all(), name
        same = torch.equal(O_ws.view(torch.int16), O_na.view(torch.int16))
        log(f"[parity] noalloc {name}: bit-identical {same}")
        assert same, name
