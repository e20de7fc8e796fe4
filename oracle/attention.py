"""Per-query sparse attention over each query's own selected pages (fp64).

What is computed ("PageWeaver: KV-Guided Query Unions for Sparse Attention",
Abstract): every query keeps its original support (its selected KV pages) and
owns its complete output; grouping queries into unions changes only the cost of
the work, never the result.  So the result of the whole path is, for each KV
head h, query (token) t and Q head hq of h:

  support   S(h, t) = { u : u = sel[h][t][s] for some slot s, 0 <= u < N }
  keys      J = { u*P + c : u in S(h, t), 0 <= c < P, u*P + c <= t }
  K^(j)     = e4m3fn(K[u][h][c][:]) * k_scale[u][h]
  V^(j)     = e4m3fn(V[u][h][c][:]) * v_scale[u][h]
  s_j       = <Q[t][hq], K^(j)> / sqrt(D)
  O[t][hq]  = sum_j softmax(s)_j V^(j)        (O = 0 when J is empty)

Readings where the pages are silent:
softmax scale 1/sqrt(D); Q head hq belongs to KV head hq // G; query t sits at
token t and sees key j iff j <= t (whole-context causal prefill); a slot value
outside [0, N) is an empty slot and repeated pages count once (the support is
a set); an empty key set gives O = 0.

``attention_groupwise`` is the union form of the same definition: each group
of query IDs evaluates every member over the union of the members' pages with a
membership-and-causal mask, which must reproduce ``attention`` (it is what the
union kernel computes, stated plainly).
"""
from __future__ import annotations

import math
import os
from typing import Optional, Sequence

import numpy as np

from .fp8 import decode_bf16, decode_e4m3fn


class Problem:
    """Decoded inputs of one call (fp64), with the shape read from the arrays."""

    def __init__(self, q_bits, k_codes, v_codes, scales, sel_pages):
        self.T, self.H_q, self.D = q_bits.shape
        self.N, self.H_kv, self.P, d2 = k_codes.shape
        assert d2 == self.D and v_codes.shape == (self.N, self.H_kv, self.P, self.D)
        assert scales.shape == (2, self.N, self.H_kv)
        assert sel_pages.shape[:2] == (self.H_kv, self.T)
        self.S = sel_pages.shape[2]
        self.G = self.H_q // self.H_kv
        self.q_bits = q_bits                               # decoded row by row
        self.k_codes, self.v_codes = k_codes, v_codes
        self.scales = np.asarray(scales, dtype=np.float64)
        self.sel = np.asarray(sel_pages)
        self._kd = {}
        self._vd = {}

    def k_hat(self, h: int) -> np.ndarray:
        """Dequantised K pages of KV head h: [N][P][D]."""
        if h not in self._kd:
            self._kd[h] = decode_e4m3fn(self.k_codes[:, h]) * self.scales[0, :, h, None, None]
        return self._kd[h]

    def v_hat(self, h: int) -> np.ndarray:
        """Dequantised V pages of KV head h: [N][P][D]."""
        if h not in self._vd:
            self._vd[h] = decode_e4m3fn(self.v_codes[:, h]) * self.scales[1, :, h, None, None]
        return self._vd[h]

    @property
    def q(self) -> np.ndarray:
        """All of Q in fp64 [T][H_q][D] (small problems)."""
        return decode_bf16(self.q_bits)

    def q_rows(self, t: int, h: int) -> np.ndarray:
        """Q[t][h*G:(h+1)*G] in fp64 [G][D]."""
        return decode_bf16(self.q_bits[t, h * self.G:(h + 1) * self.G])

    def support(self, h: int, t: int) -> np.ndarray:
        row = self.sel[h, t]
        return np.unique(row[(row >= 0) & (row < self.N)]).astype(np.int64)


def _softmax_pv(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Row-wise max-subtracted softmax of s [R][J] applied to v [J][D]."""
    if s.shape[1] == 0:
        return np.zeros((s.shape[0], v.shape[1]))
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def attention_query(pb: Problem, h: int, t: int) -> np.ndarray:
    """O[t][h*G:(h+1)*G] as fp64 [G][D]."""
    sup = pb.support(h, t)
    pos = (sup[:, None] * pb.P + np.arange(pb.P)[None, :]).ravel()
    keep = pos <= t
    kk = pb.k_hat(h)[sup].reshape(-1, pb.D)[keep]
    vv = pb.v_hat(h)[sup].reshape(-1, pb.D)[keep]
    qq = pb.q_rows(t, h)
    s = (qq @ kk.T) / math.sqrt(pb.D)
    return _softmax_pv(s, vv)


def attention_pairs(pb: Problem, pairs: Sequence[tuple]) -> np.ndarray:
    """fp64 [len(pairs)][G][D] for a list of (h, t)."""
    out = np.empty((len(pairs), pb.G, pb.D))
    for i, (h, t) in enumerate(pairs):
        out[i] = attention_query(pb, int(h), int(t))
    return out


def attention(pb: Problem) -> np.ndarray:
    """The full output O as fp64 [T][H_q][D] (single process)."""
    out = np.zeros((pb.T, pb.H_q, pb.D))
    for h in range(pb.H_kv):
        for t in range(pb.T):
            out[t, h * pb.G:(h + 1) * pb.G] = attention_query(pb, h, t)
    return out


def attention_groupwise(pb: Problem, ids: np.ndarray, g: int) -> np.ndarray:
    """Union form: O [T][H_q][D] from groups of g consecutive entries of ids[h]."""
    out = np.full((pb.T, pb.H_q, pb.D), np.nan)
    for h in range(pb.H_kv):
        for k0 in range(0, pb.T, g):
            members = [int(x) for x in ids[h, k0:k0 + g]]
            sups = [set(pb.support(h, t).tolist()) for t in members]
            union = np.array(sorted(set().union(*sups)), dtype=np.int64)
            pos = (union[:, None] * pb.P + np.arange(pb.P)[None, :]).ravel()
            page = np.repeat(union, pb.P)
            kk = pb.k_hat(h)[union].reshape(-1, pb.D)
            vv = pb.v_hat(h)[union].reshape(-1, pb.D)
            for t, sup in zip(members, sups):
                mask = np.isin(page, list(sup)) & (pos <= t)
                qq = pb.q_rows(t, h)
                s = np.where(mask[None, :], (qq @ kk.T) / math.sqrt(pb.D), -np.inf)
                if mask.any():
                    m = s.max(axis=1, keepdims=True)
                    e = np.exp(s - m)
                    o = (e @ vv) / e.sum(axis=1, keepdims=True)
                else:
                    o = np.zeros((pb.G, pb.D))
                out[t, h * pb.G:(h + 1) * pb.G] = o
    return out


# ----------------------------------------------------------------------------
# Process-pool driver (fork; the decoded Problem is shared copy-on-write).

_POOL_PB: Optional[Problem] = None


def _work(chunk):
    # one BLAS thread per worker process: the pool already uses every core
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return attention_pairs(_POOL_PB, chunk)


def attention_pairs_parallel(pb: Problem, pairs: Sequence[tuple],
                             workers: Optional[int] = None) -> np.ndarray:
    """Same as ``attention_pairs`` spread over host cores (one process each)."""
    global _POOL_PB
    workers = workers or len(os.sched_getaffinity(0))
    pairs = [(int(h), int(t)) for h, t in pairs]
    if workers <= 1 or len(pairs) < 64:
        return attention_pairs(pb, pairs)
    for h in sorted({h for h, _ in pairs}):      # decode before fork
        pb.k_hat(h)
        pb.v_hat(h)
    import multiprocessing as mp
    n_chunks = workers * 4
    chunks = [pairs[i::n_chunks] for i in range(n_chunks)]
    chunks = [c for c in chunks if c]
    _POOL_PB = pb
    try:
        pool = mp.get_context("fork").Pool(workers)
        try:
            parts = pool.map(_work, chunks)
        finally:                     # let workers exit on their own (no SIGTERM)
            pool.close()
            pool.join()
    finally:
        _POOL_PB = None
    out = np.empty((len(pairs), pb.G, pb.D))
    nc = len(chunks)
    for i, part in enumerate(parts):
        out[i::nc] = part
    return out
