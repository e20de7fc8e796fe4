"""Seeded synthetic prefill captures for query-union sparse attention.

This module produces the *inputs* of the path and nothing else: per-query
selected-page lists, bf16 queries and an FP8 (OCP e4m3fn) paged KV cache with
per-(page, KV head) fp32 scales.  It holds none of the method's arithmetic
(no grouping, no union, no attention); both the HIP path and the CPU oracle
consume what it returns.

The recorded page selections that the PageWeaver authors measured on
("PageWeaver: KV-Guided Query Unions for Sparse Attention", Abstract: the H200
results are on captured selections) are not available, so the selections are
drawn from a seeded model of the structure the AI Radio episode on the paper
describes (section "Paper summary": neighbouring query groups mix two page
communities, while queries far apart share them).

Recipe (selections: one ``numpy.random.Generator`` per KV head, seeded with
``[seed, h]``; Q/K/V normals: one ``torch.Generator`` seeded with ``seed``;
``seed = Workload.seed_for(variant)``):

* For every KV head ``h``, from its own generator:
  1. ``C`` communities, each a random subset of pages ``1..N-1`` of size
     ``M = ceil(2R/k)`` (``R = S - 1 - n_local`` community-drawn pages, ``k``
     communities per query), plus a random rank order inside each community.
  2. Segments of ``16*W`` tokens.  Per segment, ``2k`` distinct communities:
     the first ``k`` form set A, the last ``k`` set B.  Even tokens use A, odd
     tokens use B.
  3. Per (segment, parity) one matrix of uniforms, one row per query, one
     column per pool page (pool = union of the set's communities).  A query at
     page ``p = t // P`` keeps the sink page 0 and its local pages
     (``p`` and, if ``n_local == 2``, ``p-1``), then draws
     ``min(R, n - |chosen|, |valid pool|)`` pool pages ``<= p`` without
     replacement (uniform, or Zipf(a) weights ``rank**-a`` via the
     exponential race), then tops up with the highest not-yet-chosen pages
     below ``p`` until it holds ``n = min(S, p + 1)`` pages.  Rows are
     ascending and padded with -1.
* Q ~ N(0, 1) rounded to bf16 (x4 for the "peaked" variant).
* K and V ~ N(0, 1) rounded to bf16, then quantised per (page, KV head) block:
  ``scale = absmax / 448`` (1.0 for an all-zero block), codes =
  e4m3fn(x / scale) with round-to-nearest-even and saturation at +-448.

Layouts (the C-ABI layouts):
  sel_pages int32  [H_kv][T][S]
  q_bits    uint16 [T][H_q][D]        (bf16 bit patterns)
  k_codes   uint8  [N][H_kv][P][D]    (token-major page)
  v_codes   uint8  [N][H_kv][P][D]    (token-major page)
  scales    fp32   [2][N][H_kv]       (K scales, then V scales)
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch

SEED_BASE = 20261008


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens = queries (whole-context prefill, all causal)
    H_q: int
    H_kv: int
    D: int
    P: int          # page size in tokens
    S: int          # selected-page slots per (query, KV head)
    W: int          # search window
    g: int          # execution group size
    n_local: int    # local pages besides the sink
    k: int          # communities per query
    C: int          # communities per KV head
    zipf: Optional[float]
    index: int      # position in the workload table (seed offset)

    @property
    def N(self) -> int:
        return self.T // self.P

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def R(self) -> int:
        return self.S - 1 - self.n_local

    @property
    def M_comm(self) -> int:
        return -(-2 * self.R // self.k)

    @property
    def L_seg(self) -> int:
        return 16 * self.W

    def seed_for(self, variant: int = 0) -> int:
        return SEED_BASE + self.index + 16 * variant

    def shape_tuple(self):
        return (self.T, self.H_q, self.H_kv, self.D, self.P, self.N, self.S)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: tiny, then 8K / 32K / 64K prefill of a Llama-3-8B-like
# layer (32 Q / 8 KV heads, d = 128), then 64K of a 70B-like layer (GQA 8).
WORKLOADS: Dict[str, Workload] = {
    "tiny_1k": Workload("tiny_1k", 1024, 4, 1, 64, 16, 8, 32, 8, 1, 2, 8, None, 0),
    "prefill_8k": Workload("prefill_8k", 8192, 32, 8, 128, 64, 32, 64, 8, 2, 2, 16, None, 1),
    "prefill_32k": Workload("prefill_32k", 32768, 32, 8, 128, 64, 64, 128, 8, 2, 2, 32, None, 2),
    "prefill_64k": Workload("prefill_64k", 65536, 32, 8, 128, 64, 64, 256, 8, 2, 4, 64, 1.1, 3),
    "prefill_64k_70b": Workload("prefill_64k_70b", 65536, 64, 8, 128, 64, 128, 256, 8, 2, 4, 64, None, 4),
}
WORKLOAD_ORDER = list(WORKLOADS)


def _select_head(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """Selections for one KV head: int32 [T][S]."""
    T, P, S, N, R, k = wl.T, wl.P, wl.S, wl.N, wl.R, wl.k
    M = min(wl.M_comm, N - 1)
    comms = []
    for _ in range(wl.C):
        pages = rng.choice(np.arange(1, N, dtype=np.int64), size=M, replace=False)
        ranks = rng.permutation(M) + 1          # 1-based popularity rank
        comms.append((pages, ranks))
    n_seg = -(-T // wl.L_seg)
    seg_sets = [rng.choice(wl.C, size=2 * k, replace=False) for _ in range(n_seg)]

    sel = np.full((T, S), -1, dtype=np.int32)
    cols = np.arange(N, dtype=np.int64)
    for si in range(n_seg):
        t0, t1 = si * wl.L_seg, min(T, (si + 1) * wl.L_seg)
        for parity in (0, 1):
            cset = seg_sets[si][:k] if parity == 0 else seg_sets[si][k:]
            weight: Dict[int, float] = {}
            for c in cset:
                pages, ranks = comms[int(c)]
                for pg, rk in zip(pages.tolist(), ranks.tolist()):
                    w = 1.0 if wl.zipf is None else float(rk) ** (-wl.zipf)
                    weight[pg] = max(weight.get(pg, 0.0), w)
            pool = np.array(sorted(weight), dtype=np.int64)
            wts = np.array([weight[x] for x in pool.tolist()], dtype=np.float64)
            ts = np.arange(t0 + parity, t1, 2, dtype=np.int64)
            if ts.size == 0:
                continue
            u = rng.random((ts.size, pool.size))
            p = ts // P
            n = np.minimum(S, p + 1)
            chosen = np.zeros((ts.size, N), dtype=bool)
            rows = np.arange(ts.size)
            chosen[:, 0] = True
            chosen[rows, p] = True
            if wl.n_local >= 2:
                chosen[rows, np.maximum(p - 1, 0)] = True
            n_chosen = chosen.sum(axis=1)
            valid = (pool[None, :] <= p[:, None]) & ~chosen[:, pool]
            if wl.zipf is None:
                key = u
            else:   # exponential race: smallest Exp(1)/w first
                key = -np.log1p(-u) / wts[None, :]
            key = np.where(valid, key, np.inf)
            order = np.argsort(key, axis=1, kind="stable")
            draws = np.minimum(np.minimum(wl.R, n - n_chosen), valid.sum(axis=1))
            take = np.arange(pool.size)[None, :] < draws[:, None]
            rr, cc = np.nonzero(take)
            chosen[rr, pool[order[rr, cc]]] = True
            # top-up: highest pages below p that are not chosen yet
            need = n - chosen.sum(axis=1)
            free = (~chosen) & (cols[None, :] < p[:, None])
            from_top = np.cumsum(free[:, ::-1], axis=1)[:, ::-1]
            chosen |= free & (from_top <= need[:, None])
            cnt = chosen.sum(axis=1)
            assert np.array_equal(cnt, n), "top-up failed"
            # ascending page lists, padded with -1
            srt = np.argsort(~chosen, axis=1, kind="stable")[:, :S]
            keep = np.arange(S)[None, :] < n[:, None]
            sel[ts] = np.where(keep, srt, -1).astype(np.int32)
    return sel


def _select_head_seeded(args):
    wl, seed, h = args
    return _select_head(wl, np.random.default_rng([seed, h]))


def make_selection(wl: Workload, variant: int = 0, workers: int = 0) -> np.ndarray:
    """int32 [H_kv][T][S] selected pages (ascending, -1 padded).

    ``workers > 1`` generates the heads in a process pool (same result)."""
    jobs = [(wl, wl.seed_for(variant), h) for h in range(wl.H_kv)]
    if workers > 1 and wl.H_kv > 1:
        import multiprocessing as mp
        pool = mp.get_context("fork").Pool(min(workers, wl.H_kv))
        try:
            heads = pool.map(_select_head_seeded, jobs)
        finally:                     # let workers exit on their own (no SIGTERM)
            pool.close()
            pool.join()
    else:
        heads = [_select_head_seeded(j) for j in jobs]
    return np.stack(heads, axis=0)


def _quantise_blocks(x_bf16: torch.Tensor):
    """x: bf16 [N][H][P][D] -> (codes uint8 same shape, scales fp32 [N][H])."""
    xf = x_bf16.float()
    amax = xf.abs().amax(dim=(2, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (xf / scale[:, :, None, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_qkv(wl: Workload, variant: int = 0, peaked: bool = False):
    """bf16 Q bits and an e4m3fn paged KV cache (numpy arrays, C-ABI layouts)."""
    gen = torch.Generator().manual_seed(wl.seed_for(variant))
    q = torch.randn((wl.T, wl.H_q, wl.D), generator=gen).to(torch.bfloat16)
    if peaked:
        q = q * 4
    k = torch.randn((wl.N, wl.H_kv, wl.P, wl.D), generator=gen).to(torch.bfloat16)
    v = torch.randn((wl.N, wl.H_kv, wl.P, wl.D), generator=gen).to(torch.bfloat16)
    kc, ks = _quantise_blocks(k)
    vc, vs = _quantise_blocks(v)
    scales = torch.stack([ks, vs], dim=0).contiguous()
    return {
        "q_bits": q.view(torch.int16).numpy().view(np.uint16),
        "k_codes": kc.numpy(),
        "v_codes": vc.numpy(),
        "scales": scales.numpy().astype(np.float32),
    }


def make_inputs(wl: Workload, variant: int = 0, peaked: bool = False) -> dict:
    d = make_qkv(wl, variant, peaked)
    d["sel_pages"] = make_selection(wl, variant)
    return d


def identity_ids(wl: Workload) -> np.ndarray:
    """Adjacent grouping: every KV head keeps token order (no search)."""
    return np.tile(np.arange(wl.T, dtype=np.int32), (wl.H_kv, 1))


def support_sizes(sel: np.ndarray, N: int) -> np.ndarray:
    """|support| per (head, query): distinct in-range entries of each row."""
    valid = (sel >= 0) & (sel < N)
    s = np.sort(np.where(valid, sel, -1), axis=2)
    distinct = s >= 0
    distinct[:, :, 1:] &= s[:, :, 1:] != s[:, :, :-1]
    return distinct.sum(axis=2)


def useful_flops(sel: np.ndarray, wl: Workload) -> float:
    """4*D flops per (visible selected key, Q head): QK^T and PV, own support only.

    Rows must hold distinct pages (the generator's rows do)."""
    H, T, S = sel.shape
    t = np.arange(T, dtype=np.int64)
    vis = np.zeros((H, T), dtype=np.int64)
    for s_ in range(S):
        u = sel[:, :, s_].astype(np.int64)
        ok = (u >= 0) & (u < wl.N)
        keys = np.clip(t[None, :] - u * wl.P + 1, 0, wl.P)
        vis += np.where(ok, keys, 0)
    return float(vis.sum()) * wl.G * 4 * wl.D
