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
from typing import Sequence

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


def attention_query_lowp(pb: Problem, h: int, t: int, tau: float = TAU) -> np.ndarray:
    """O[t][h*G:(h+1)*G] of the low-precision variant as fp64 [G][D]."""
    out = np.zeros((pb.G, pb.D))
    sup = pb.support(h, t)                  # ascending, each page once
    qq = pb.q_rows(t, h)
    kc = decode_e4m3fn(pb.k_codes[:, h])    # [N][P][D] codes
    vc = decode_e4m3fn(pb.v_codes[:, h])
    c = math.log2(math.e) / math.sqrt(pb.D)
    for r in range(pb.G):
        qt = quantize_q_row(qq[r])
        m = -math.inf
        num = np.zeros(pb.D)
        den = 0.0
        for u in sup:
            u = int(u)
            keys = [j for j in range(pb.P) if u * pb.P + j <= t]
            if not keys:
                continue
            s = (kc[u, keys] @ qt) * pb.scales[0, u, h] * c
            mx = float(s.max())
            if mx > m + tau:                # the reference moves (step 3)
                if m > -math.inf:
                    num *= 2.0 ** (m - mx)
                    den *= 2.0 ** (m - mx)
                m = mx
            phi, k = split_scale(float(pb.scales[1, u, h]))
            p = e4m3_rne(np.exp2(s - m) * phi)
            num += 2.0 ** k * (p @ vc[u, keys])
            den += float(p.sum()) / phi
        if den > 0.0:
            out[r] = num / den
    return out


def attention_pairs_lowp(pb: Problem, pairs: Sequence[tuple], tau: float = TAU) -> np.ndarray:
    """fp64 [len(pairs)][G][D] of the variant for a list of (h, t)."""
    out = np.empty((len(pairs), pb.G, pb.D))
    for i, (h, t) in enumerate(pairs):
        out[i] = attention_query_lowp(pb, int(h), int(t), tau)
    return out
