"""The FP8 Q and P variant's parity gate (tests/fp8qp_gate.py) on the CPU: it accepts the model
itself and a model that rounds ties of p the other way (the kind of difference the kernel's own
scores cause), and it rejects planted errors."""
import numpy as np
import pytest

import oracle.lowp as lowp
from tests.fp8qp_gate import assert_close_lowp, model_rows
from tests.gpu_common import problem
from tests.oracle_helpers import tiny_problem


def _bf16(x):
    """Round fp64 values to bf16 (nearest even) as the kernel's output is."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    f = (f + 0x7FFF + ((f >> 16) & 1)) & 0xFFFF0000
    return f.astype(np.uint32).view(np.float32).astype(np.float64)


def _inputs():
    # peaked rows, and V scales 17/16 * 2^k on every third page: each such page's largest key
    # has x = phi = 17/16 exactly, a rounding midpoint of e4m3fn
    inp = tiny_problem(T=256, Hq=8, Hkv=2, D=64, P=16, S=6, seed=11, q_scale=4.0)
    sc = inp["scales"].copy()
    pages = np.arange(0, sc.shape[1], 3)
    sc[1, pages] = ((17 / 16) * 2.0 ** (pages % 4 - 2))[:, None]     # 17/16 times 1/4 .. 2
    return dict(inp, scales=sc.astype(np.float32))


def _pairs(inp):
    return [(h, t) for h in range(inp["sel_pages"].shape[0]) for t in range(inp["q_bits"].shape[0])]


def _tie_up(x):
    """Nearest e4m3fn value with ties to the larger magnitude."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    pos = lowp._POS
    hi = np.minimum(np.searchsorted(pos, a, side="left"), len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (pos[hi] - a) <= (a - pos[lo])
    return np.copysign(np.where(a == pos[hi], pos[hi], np.where(pick_hi, pos[hi], pos[lo])), x)


@pytest.fixture(scope="module")
def case():
    inp = _inputs()
    pairs = _pairs(inp)
    model = model_rows(inp, pairs)
    return inp, pairs, model


def test_accepts_the_model_rounded_to_bf16(case):
    inp, pairs, model = case
    assert_close_lowp(_bf16(model[0]), model, "model itself")


def test_accepts_ties_rounded_the_other_way(case, monkeypatch):
    inp, pairs, model = case
    rne = lowp.e4m3_rne
    # only the rounding of p changes: q keeps round-to-nearest-even, as on the GPU
    monkeypatch.setattr(lowp, "quantize_q_row",
                        lambda q: rne(np.ldexp(q, lowp.row_exponent(q))) * 2.0 ** -lowp.row_exponent(q))
    monkeypatch.setattr(lowp, "e4m3_rne", _tie_up)
    pb = problem(inp)
    alt = np.stack([lowp.attention_query_lowp(pb, h, t) for h, t in pairs])
    monkeypatch.undo()
    assert np.abs(alt - model[0]).max() > 1e-3            # the tie rule does change rows
    assert_close_lowp(_bf16(alt), model, "ties the other way")


@pytest.mark.parametrize("kind", ["one element", "scale", "dropped key"])
def test_rejects_planted_errors(case, kind):
    inp, pairs, model = case
    ref, allow, und = model
    got = _bf16(ref).copy()
    if kind == "one element":
        i, r, d = np.unravel_index(np.argmin(allow), allow.shape)
        got[i, r, d] += 0.05
    elif kind == "scale":
        got *= 1.03
    else:                                   # one row computed without the query's own page
        pb = problem(inp)
        h, t = pairs[-1]
        sel = inp["sel_pages"].copy()
        row = sel[h, t]
        row[row == t // pb.P] = -1                          # drop the query's own page
        pb2 = problem(dict(inp, sel_pages=sel))
        got[len(pairs) - 1] = _bf16(lowp.attention_query_lowp(pb2, h, t))
    with pytest.raises(AssertionError):
        assert_close_lowp(got, model, f"planted {kind}")
