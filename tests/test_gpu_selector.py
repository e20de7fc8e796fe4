"""pw_select on the GPU against the selector oracle.

The fixed pages, row sizes, order, padding and causality are compared
exactly.  The chosen pages are a top-k decided by floating-point scores: the
kernel ranks fp32 scores computed on the matrix cores from bf16 hi/lo parts,
the oracle exact fp64 ones, so pages within the kernel's error bound of the
k-th score may go either way.  Each row must therefore be a valid top-k
within that bound (everything clearly above the threshold chosen, nothing
clearly below it), and rows are reported that differ from the oracle at all.
"""
import numpy as np
import pytest
import torch

from oracle.selector import fixed_pages, query_sums, key_sums
from query_union_paged_amd import synth
from tests.gpu_common import assert_close, gpu_rows, log, oracle_rows

pytestmark = pytest.mark.gpu
REL = 2.0 ** -12          # score error bound, relative to ks * sum_d |qs_d C_d| (actual ~2^-16)


def _pw():
    from query_union_paged_amd import pageweaver
    return pageweaver


def _problem(T, Hq, Hkv, D, P, seed):
    N = T // P
    gen = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = torch.randn((T, Hq, D), generator=gen).to(torch.bfloat16)
    k = torch.randn((N, Hkv, P, D), generator=gen).to(torch.float8_e4m3fn)
    return {"q_bits": q.view(torch.int16).numpy().view(np.uint16), "k_codes": k.view(torch.uint8).numpy(),
            "scales": rng.uniform(0.05, 1.0, size=(2, N, Hkv)).astype(np.float32)}


def _run(inp, S, L, reps=1):
    pw = _pw()
    T, Hq, D = inp["q_bits"].shape
    N, Hkv, P, _ = inp["k_codes"].shape
    shp = pw.shape(T, Hq, Hkv, D, P, N, S)
    dev = pw.to_device({k: inp[k] for k in ("q_bits", "k_codes", "scales")})
    outs = [pw.pw_select(shp, dev["q_bits"], dev["k_codes"], dev["scales"], L) for _ in range(reps)]
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _check_rows(inp, sel, S, L, rows=None):
    """Exact structure + top-k validity within the error bound; returns rows unlike the oracle's."""
    T, Hq, D = inp["q_bits"].shape
    N, Hkv, P, _ = inp["k_codes"].shape
    G = Hq // Hkv
    rows = range(T) if rows is None else rows
    differ = 0
    for h in range(Hkv):
        qs = query_sums(inp["q_bits"], h, G)
        C = key_sums(inp["k_codes"], h)
        ks = inp["scales"][0][:, h].astype(np.float64)
        for t in rows:
            p = t // P
            row = sel[h, t]
            got = row[row >= 0]
            fixed = fixed_pages(p, L)
            cand = [u for u in range(1, p + 1) if u not in set(fixed)]
            k = min(S - len(fixed), len(cand))
            assert np.all(np.diff(got) > 0) and np.all(row[got.size:] == -1), (h, t, row)
            assert got.size == len(fixed) + k and set(fixed) <= set(got.tolist()), (h, t, row)
            chosen = sorted(set(got.tolist()) - set(fixed))
            assert set(chosen) <= set(cand), (h, t, row)
            if k == 0 or k == len(cand):
                continue
            c = np.array(cand)
            s = ks[c] * (C[c] @ qs[t])
            bound = ks[c] * (np.abs(C[c]) @ np.abs(qs[t])) * REL
            order = sorted(range(len(c)), key=lambda i: (-s[i], c[i]))
            thr = s[order[k - 1]]
            pick = np.isin(c, chosen)
            eps = 2 * bound.max()
            assert s[pick].min() >= thr - eps and s[~pick].max() <= thr + eps, (h, t)
            differ += int(set(c[order[:k]].tolist()) != set(chosen))
    return differ


@pytest.mark.parametrize("T,Hq,Hkv,D,P,S,L", [
    (1024, 4, 1, 64, 16, 8, 1), (2048, 8, 2, 128, 32, 12, 2), (4096, 32, 8, 128, 64, 16, 2),
    (4096, 2, 1, 64, 16, 40, 3), (1024, 8, 1, 128, 64, 4, 3)])
def test_selector_parity(T, Hq, Hkv, D, P, S, L):
    log(f"[case] pw_select T={T} Hq={Hq} Hkv={Hkv} D={D} P={P} S={S} L={L}")
    inp = _problem(T, Hq, Hkv, D, P, seed=T + S + L)
    sel, again = _run(inp, S, L, reps=2)
    assert np.array_equal(sel, again)                      # deterministic
    differ = _check_rows(inp, sel, S, L)
    log(f"[parity] pw_select rows unlike the oracle (near-ties): {differ} of {T * Hkv}")
    assert differ <= max(2, T * Hkv // 1000)


def test_selector_largest_pages_and_pipeline():
    # N = 1024 pages (the limit) at the 64K workload's shape; sampled rows against the oracle,
    # then the selections feed the search and the union attention
    wl = synth.WORKLOADS["prefill_64k"]
    log("[case] pw_select prefill_64k shape, then pw_group and pw_union_attention")
    inp = synth.make_qkv(wl)
    sel, = _run(inp, wl.S, 2)
    rng = np.random.default_rng(3)
    rows = sorted(set(range(64)) | set(range(wl.T - 64, wl.T)) |
                  set(rng.choice(wl.T, size=64, replace=False).tolist()))
    differ = _check_rows(inp, sel, wl.S, 2, rows)
    log(f"[parity] pw_select 64K sample: {differ} of {len(rows) * wl.H_kv} rows unlike the oracle")
    assert differ <= 2
    pw = _pw()
    full = dict(inp, sel_pages=sel)
    dev = pw.to_device(full)
    shp = pw.shape(*wl.shape_tuple())
    ids = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    O = pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, wl.g)
    torch.cuda.synchronize()
    pairs = [(h, t) for h in range(wl.H_kv) for t in rows[::4]]
    assert_close(gpu_rows(O, pairs, wl.G), oracle_rows(full, pairs), "attention on selector output")


def test_selector_invalid_arguments():
    pw = _pw()
    inp = _problem(256, 4, 1, 64, 16, 1)
    dev = pw.to_device(inp)
    for S, L in [(4, 0), (4, 4)]:
        shp = pw.shape(256, 4, 1, 64, 16, 16, S)
        with pytest.raises(pw.PWError) as e:
            pw.pw_select(shp, dev["q_bits"], dev["k_codes"], dev["scales"], L)
        assert e.value.status == pw.PW_ERR_UNSUPPORTED
