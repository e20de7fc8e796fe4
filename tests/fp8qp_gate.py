"""Parity gate of the FP8 Q and P variant against its fp64 model (oracle.lowp): the model's
rows, a per-element rounding-flip allowance from the model's per-page trace, and the check.
Used by the GPU tests of pw_union_attention_tiled_fp8qp and pinned on the CPU."""
import math
import time

import numpy as np

from oracle.fp8 import E4M3FN_TABLE
from oracle.lowp import TAU, _codes, attention_query_lowp, quantize_q_row
from tests.gpu_common import TOL_MAX, TOL_MEAN, TOL_REL_RMS, WORKERS, errors, log, problem

# The model rounds p = 2^(s - m) phi to e4m3fn from exact arguments, the kernel from its own
# scores: the FP8 MFMA accumulates with an error of up to 3.8e-5 of the sum of the products'
# magnitudes (measured: 2048 random 32x32x64 tiles of workload-like operands, median 1.2e-6),
# plus fp32 rounding and the hardware exp2.  Where an argument lies within that error of a
# rounding midpoint (always, for the page maximum of a page whose V scale mantissa phi is itself
# a midpoint, such as 17/16), the two round to neighbouring e4m3fn values.  The check therefore
# replays the model (its per-page trace), flags every key whose x lies within the error window
# of a midpoint, and allows each flagged key one rounding step of its weight times |v - O|.
# Gates: the error left after each element's allowance meets the exact path's bounds (max,
# mean and relative RMS).  A row whose reference move itself lies within the
# error window of the threshold (either choice is correct, and the two round every later p at
# different points) is allowed one rounding step on every key instead, and such rows stay rare.
MFMA_REL = 2.0 ** -14       # bound on the FP8 MFMA's accumulation error / sum |products|
FP32_REL = 2.0 ** -20       # fp32 arguments and exp2, relative to the magnitudes involved
UNDECIDED_FRACTION = 1e-2
LOG2E = math.log2(math.e)
_POS = np.unique(np.abs(E4M3FN_TABLE[np.isfinite(E4M3FN_TABLE)]))


def flip_allowance(pb, h, t):
    """(O, allowance [G][D], undecided [G]) of one query of the model (see above); an
    undecided row's allowance counts one rounding step on every key."""
    tr = []
    O = attention_query_lowp(pb, h, t, trace=tr)
    allow = np.zeros((pb.G, pb.D))
    undecided = np.zeros(pb.G, dtype=bool)
    if not tr:
        return O, allow, undecided
    kc, vc = _codes(pb, h)
    qt = np.stack([quantize_q_row(q) for q in pb.q_rows(t, h)])
    c = LOG2E / math.sqrt(pb.D)
    m_fin = tr[-1]["m"]
    den = sum(np.exp2(e["m"] - m_fin) * e["p"].sum(axis=1) / e["phi"] for e in tr)
    d_m = np.zeros(pb.G)                     # error bound of the current reference
    flip_w = np.zeros(pb.G)
    allow_all = np.zeros((pb.G, pb.D))
    all_w = np.zeros(pb.G)
    for e in tr:
        u, nk = e["u"], e["nk"]
        absum = (np.abs(qt) @ np.abs(kc[u, :nk]).T) * pb.scales[0, u, h] * c
        d_s = MFMA_REL * absum + FP32_REL * (np.abs(e["s"]) + 8)
        d_page = d_s.max(axis=1)
        moved = e["m"] != e["m_in"]
        known = np.isfinite(e["m_in"])
        undecided |= known & (np.abs(e["mx"] - e["m_in"] - TAU) <= d_page + d_m)
        d_m = np.where(moved, d_page, d_m)
        win = math.log(2) * (d_s + d_m[:, None] + FP32_REL * (np.abs(e["m"])[:, None] + 8))
        x = e["x"]
        i = np.clip(np.searchsorted(_POS, x, side="right"), 1, len(_POS) - 1)
        lo, hi = _POS[i - 1], _POS[i]
        step = np.where(x == lo, 0.0, hi - lo)
        flagged = np.abs(x - (lo + hi) / 2) <= win * x
        w_all = (np.exp2(e["m"] - m_fin) / e["phi"] / den)[:, None] * step          # [G][nk]
        w = w_all * flagged
        dev = np.abs(vc[u, :nk][None] * pb.scales[1, u, h] - O[:, None, :])         # [G][nk][D]
        allow += np.einsum("rj,rjd->rd", w, dev)
        allow_all += np.einsum("rj,rjd->rd", w_all, dev)
        flip_w += w.sum(axis=1)
        all_w += w_all.sum(axis=1)
    allow /= np.maximum(1.0 - np.minimum(flip_w, 0.5), 0.5)[:, None]
    allow_all /= np.maximum(1.0 - np.minimum(all_w, 0.5), 0.5)[:, None]
    allow = np.where(undecided[:, None], allow_all, allow)
    return O, allow, undecided


_POOL = None


def _allow_chunk(chunk):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return [flip_allowance(_POOL, h, t) for h, t in chunk]


def model_rows(inp, pairs):
    """The model's rows, allowances and undecided flags for (h, t) pairs (process pool)."""
    global _POOL
    t0 = time.time()
    pb = problem(inp)
    pairs = [(int(h), int(t)) for h, t in pairs]
    for h in sorted({h for h, _ in pairs}):
        _codes(pb, h)
    n = max(1, min(WORKERS * 4, len(pairs)))
    chunks = [pairs[i::n] for i in range(n)]
    _POOL = pb
    try:
        if WORKERS > 1 and len(pairs) >= 64:
            import multiprocessing as mp
            pool = mp.get_context("fork").Pool(WORKERS)
            try:
                parts = pool.map(_allow_chunk, chunks)
            finally:
                pool.close()
                pool.join()
        else:
            parts = [_allow_chunk(c) for c in chunks]
    finally:
        _POOL = None
    res = [None] * len(pairs)
    for k, part in enumerate(parts):
        res[k::n] = part
    O = np.stack([r[0] for r in res])
    allow = np.stack([r[1] for r in res])
    und = np.stack([r[2] for r in res])
    log(f"[oracle] fp8 model + flip allowance: {len(pairs)} (head, query) rows in "
        f"{time.time() - t0:.1f}s")
    return O, allow, und


def assert_close_lowp(got, model, what=""):
    """The error left after each element's flip allowance must meet the exact path's bounds:
    max 2e-2, mean 2e-3 and relative RMS 5e-3 (the raw errors are logged beside it)."""
    ref, allow, und = model
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e = errors(got, ref)
    diff = np.abs(got - ref)
    excess = np.maximum(diff - allow, 0.0)
    ex = {"max": float(excess.max()), "mean": float(excess.mean()),
          "rel_rms": float(np.sqrt((excess ** 2).sum() / max((ref ** 2).sum(), 1e-300)))}
    bad = (excess > TOL_MAX).any(axis=2)
    frac_und = float(und.mean())
    n_allow = int(((diff > TOL_MAX) & ~(excess > TOL_MAX)).any(axis=2).sum())
    log(f"[parity] {what}: max {e['max']:.3e} mean {e['mean']:.3e} rel_rms {e['rel_rms']:.3e}; "
        f"beyond the flip allowance: max {ex['max']:.3e} mean {ex['mean']:.3e} rel_rms "
        f"{ex['rel_rms']:.3e}; rows above {TOL_MAX} within their allowance: {n_allow}, undecided "
        f"rows {frac_und:.2e}")
    assert ex["mean"] <= TOL_MEAN and ex["rel_rms"] <= TOL_REL_RMS, f"{what}: {ex}"
    assert frac_und <= UNDECIDED_FRACTION, f"{what}: {frac_und} undecided rows"
    assert not bad.any(), f"{what}: {int(bad.sum())} rows outside bound + allowance"
    return e
