"""A synthetic dynamic page selector (the step that produces ``sel_pages``).

The pages start from dynamic sparse attention: every query has its own set of
selected KV pages ("PageWeaver: KV-Guided Query Unions for Sparse Attention",
Abstract).  How the set is chosen is not part of the method, so this is a
stand-in of our own, in the common block-sparse style, used to feed the path
with selections derived from Q and K instead of drawn communities.

Definition (per KV head h and query t, own page p = t // P):

* fixed pages: page 0 (the sink) and the L local pages p, p-1, ..., p-L+1
  (those >= 0);
* candidates: pages 1..p that are not fixed;
* score of page u:  ks[u][h] * sum_d qs_t[d] * C_u[d], where qs_t is the sum
  of the query's G head rows of that KV head and C_u[d] the sum over the
  page's P keys of the dequantised-before-scale K codes (the page's key
  "centre", up to the factor P);
* the min(S - |fixed|, |candidates|) candidates with the largest score are
  chosen; ties go to the lower page;
* the row is fixed + chosen in ascending page order, padded with -1 to S.

Here every quantity is exact or fp64: C_u is an exact sum of e4m3 values,
qs_t a sum of bf16 values in fp64, and the score a single fp64 dot product.
TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .fp8 import decode_bf16, decode_e4m3fn


def fixed_pages(p: int, L: int) -> list:
    """Sink and local pages of a query on page p, ascending, without repeats."""
    return sorted({0} | {p - i for i in range(L) if p - i >= 0})


def key_sums(k_codes: np.ndarray, h: int) -> np.ndarray:
    """C[u][d] = sum over the page's keys of e4m3(K[u][h][j][d]), fp64 [N][D]."""
    return decode_e4m3fn(k_codes[:, h]).sum(axis=1)


def query_sums(q_bits: np.ndarray, h: int, G: int) -> np.ndarray:
    """qs[t][d] = sum of the G query rows of KV head h, fp64 [T][D]."""
    return decode_bf16(q_bits[:, h * G:(h + 1) * G]).sum(axis=1)


def scores(q_bits, k_codes, scales, h: int, G: int, rows=None) -> np.ndarray:
    """fp64 page scores [len(rows)][N] for KV head h (all queries if rows is None)."""
    qs = query_sums(q_bits, h, G)
    if rows is not None:
        qs = qs[np.asarray(rows)]
    C = key_sums(k_codes, h)
    return (qs @ C.T) * scales[0][:, h].astype(np.float64)[None, :]


def select_row(score_row: np.ndarray, p: int, S: int, L: int) -> np.ndarray:
    """One selection row from the scores of pages 0..N-1 (only pages <= p are used)."""
    fixed = fixed_pages(p, L)
    cand = [u for u in range(1, p + 1) if u not in set(fixed)]
    k = min(S - len(fixed), len(cand))
    # largest score first, then the lower page
    order = sorted(cand, key=lambda u: (-score_row[u], u))
    chosen = order[:k]
    row = sorted(fixed + chosen)
    return np.array(row + [-1] * (S - len(row)), dtype=np.int32)


def select(q_bits, k_codes, scales, S: int, L: int, P: int, rows=None, heads=None) -> dict:
    """Selections {(h, t): row} for the given queries (default: all) and KV heads."""
    T, Hq, _ = q_bits.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    rows = list(range(T)) if rows is None else list(rows)
    heads = list(range(Hkv)) if heads is None else list(heads)
    out = {}
    for h in heads:
        sc = scores(q_bits, k_codes, scales, h, G, rows)
        for i, t in enumerate(rows):
            out[(h, t)] = select_row(sc[i], t // P, S, L)
    return out
