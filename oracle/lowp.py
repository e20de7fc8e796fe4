"""Low-precision variant of the union attention: Q and P in e4m3fn (fp64 model).

Test infrastructure only: tests, the smoke check and the CPU leg of the benchmark
may call this module; the library never does.

The pages fix the KV cache as FP8 ("PageWeaver: KV-Guided Query Unions for
Sparse Attention", Abstract) and say nothing about the precision of Q or of the
softmax probabilities P.  The exact path keeps both at bf16 accuracy.  The
library also offers an opt-in variant in the style of FlashAttention-3's FP8
mode (the mlsanity page on the paper, "Builds on") in which Q and P are
quantised per row to e4m3fn, so that both products run on the FP8 matrix cores.
This module is that variant's definition, step by step, in fp64.  The GPU
variant is compared with it, and it is compared with the exact attention
(``oracle.attention``) to state what the variant costs in accuracy.

Definition, per KV head h, query (token) t and Q head hq of h, with the support,
the visible keys and the decoded K codes as in ``oracle.attention``:

 1. Row scaling of q (the bf16 row): e = 8 - x where max_i |q_i| = f 2^x,
    f in [1/2, 1) (e = 0 for a zero row), so that max |q| 2^e lies in [128, 256);
    q_hat = rne(q 2^e) and q~ = q_hat 2^-e, with rne the rounding to the nearest
    e4m3fn value, ties to the even code.
 2. The row's support pages in ascending page order; on page u the scores of
    its visible keys j in log2 units:
        s_j = <q~, K_codes[j]> k_scale_u log2(e) / sqrt(D).
 3. A reference maximum m, -inf at the start: when the largest s_j of a page
    exceeds m + tau (tau = 6) it becomes the new m, and what was summed so far is
    multiplied by 2^(m_old - m_new).
 4. v_scale_u = phi_u 2^k_u with phi_u in [1, 2) and k_u an integer;
        p_j = rne(2^(s_j - m) phi_u)          (at most 2^(tau + 1) = 128)
 5. num += 2^k_u sum_j p_j V_codes[j]          den += sum_j p_j / phi_u
 6. O = num / den, and O = 0 when the row sees no key.

Since p_j / phi_u is 2^(s_j - m) up to the rounding, O is the exact softmax
average of v_scale * V_codes up to the e4m3 rounding of q and p.
"""
from __future__ import annotations

import math
import os
from typing import Optional, Sequence

import numpy as np

from .attention import Problem
from .fp8 import E4M3FN_TABLE, decode_e4m3fn

TAU = 6.0

# the finite non-negative e4m3fn values in code order (codes 0x00 .. 0x7E)
_POS = E4M3FN_TABLE[:0x7F].copy()


def e4m3_rne(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest e4m3fn value, ties to the even code.

    Magnitudes up to 448 only (every value this module rounds stays below 2^8);
    the sign is kept, and zero stays zero."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448.0) or np.any(np.isnan(a)):
        raise ValueError("e4m3_rne: magnitude above 448 or NaN")
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == _POS[hi], hi, np.where(pick_hi, hi, lo))
    return np.copysign(_POS[code], x)


def row_exponent(q: np.ndarray) -> int:
    """e of step 1 for one row (0 for a zero row)."""
    amax = float(np.max(np.abs(q))) if q.size else 0.0
    if amax == 0.0:
        return 0
    _, x = math.frexp(amax)                 # amax = f 2^x, f in [1/2, 1)
    return 8 - x


def quantize_q_row(q: np.ndarray) -> np.ndarray:
    """q~ of step 1 (fp64, the dequantised e4m3fn row)."""
    e = row_exponent(q)
    return e4m3_rne(np.ldexp(q, e)) * 2.0 ** (-e)


def split_scale(v_scale: float):
    """(phi, k) with v_scale = phi 2^k, phi in [1, 2) (v_scale > 0)."""
    f, x = math.frexp(v_scale)              # v_scale = f 2^x, f in [1/2, 1)
    return 2.0 * f, x - 1


def _codes(pb: Problem, h: int):
    """Decoded K and V codes of KV head h, [N][P][D] each (cached on the problem)."""
    cache = pb.__dict__.setdefault("_lowp_codes", {})
    if h not in cache:
        cache[h] = (decode_e4m3fn(pb.k_codes[:, h]), decode_e4m3fn(pb.v_codes[:, h]))
    return cache[h]


def attention_query_lowp(pb: Problem, h: int, t: int, tau: float = TAU,
                         trace: Optional[list] = None) -> np.ndarray:
    """O[t][h*G:(h+1)*G] of the low-precision variant as fp64 [G][D] (the G rows of the
    query side by side; each keeps its own reference maximum).  With a list as `trace`,
    every page appends its intermediate values: u, nk (visible keys), the reference m
    before and after the page (m_in, m), the page maxima mx and the scores s, the
    unrounded x = 2^(s - m) phi and the rounded p, phi and k."""
    out = np.zeros((pb.G, pb.D))
    sup = pb.support(h, t)                  # ascending, each page once
    sup = sup[sup * pb.P <= t]              # pages with at least one visible key
    if sup.size == 0:
        return out
    kc, vc = _codes(pb, h)
    qt = np.stack([quantize_q_row(q) for q in pb.q_rows(t, h)])     # [G][D]
    c = math.log2(math.e) / math.sqrt(pb.D)
    m = np.full(pb.G, -np.inf)
    num = np.zeros((pb.G, pb.D))
    den = np.zeros(pb.G)
    for u in sup:
        u = int(u)
        nk = min(pb.P, t - u * pb.P + 1)    # visible keys 0 .. nk - 1
        s = (qt @ kc[u, :nk].T) * pb.scales[0, u, h] * c           # [G][nk]
        mx = s.max(axis=1)
        move = mx > m + tau                 # the reference moves (step 3)
        f = np.where(move & (m > -np.inf), np.exp2(np.where(move, m - mx, 0.0)), 1.0)
        num *= f[:, None]
        den *= f
        m_in, m = m, np.where(move, mx, m)
        phi, k = split_scale(float(pb.scales[1, u, h]))
        x = np.exp2(s - m[:, None]) * phi
        p = e4m3_rne(x)
        num += 2.0 ** k * (p @ vc[u, :nk])
        den += p.sum(axis=1) / phi
        if trace is not None:
            trace.append({"u": u, "nk": nk, "m_in": m_in, "m": m, "mx": mx, "s": s, "x": x,
                          "p": p, "phi": phi, "k": k})
    return num / den[:, None]


def attention_pairs_lowp(pb: Problem, pairs: Sequence[tuple], tau: float = TAU) -> np.ndarray:
    """fp64 [len(pairs)][G][D] of the variant for a list of (h, t)."""
    out = np.empty((len(pairs), pb.G, pb.D))
    for i, (h, t) in enumerate(pairs):
        out[i] = attention_query_lowp(pb, int(h), int(t), tau)
    return out


# ----------------------------------------------------------------------------
# Process-pool driver (fork; the decoded Problem is shared copy-on-write).

_POOL_PB: Optional[Problem] = None


def _work(chunk):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return attention_pairs_lowp(_POOL_PB, chunk)


def attention_pairs_lowp_parallel(pb: Problem, pairs: Sequence[tuple],
                                  workers: Optional[int] = None) -> np.ndarray:
    """Same as ``attention_pairs_lowp`` spread over host cores (one process each)."""
    global _POOL_PB
    workers = workers or len(os.sched_getaffinity(0))
    pairs = [(int(h), int(t)) for h, t in pairs]
    if workers <= 1 or len(pairs) < 64:
        return attention_pairs_lowp(pb, pairs)
    for h in sorted({h for h, _ in pairs}):      # decode before fork
        _codes(pb, h)
    import multiprocessing as mp
    n_chunks = workers * 4
    chunks = [c for c in (pairs[i::n_chunks] for i in range(n_chunks)) if c]
    _POOL_PB = pb
    try:
        pool = mp.get_context("fork").Pool(workers)
        try:
            parts = pool.map(_work, chunks)
        finally:
            pool.close()
            pool.join()
    finally:
        _POOL_PB = None
    out = np.empty((len(pairs), pb.G, pb.D))
    for i, part in enumerate(parts):
        out[i::len(chunks)] = part
    return out
