"""Complete-call benchmark of query-union sparse-attention prefill on one MI355X.

One step = one complete call on resident inputs: the grouping search with its
group order (pw_group_ordered), the re-tiling of the FP8 pages (pw_tile_kv) and
the union attention in that order (pw_union_attention_tiled_ordered), all on one
stream, each bracketed by HIP events.  The same call in the search's own group
order (pw_group + pw_union_attention_tiled, bit-identical output) is an arm.
Every timed step is cold: a 1 GiB buffer is written before it (outside its
events), which evicts the MALL and the L2.  Warm steps (no flush) are reported
beside it.  Default workload: 64K-token prefill of a Llama-3-8B-like layer
(32 Q / 8 KV heads, d = 128, page 64, 64 selected pages per (query, KV head),
Zipf(1.1) community draws, W = 256, g = 8), FP8 e4m3fn KV, bf16 Q and O.

Prints one JSON line.  `value` is useful TFLOP/s of the cold complete call:
4*D flops per (visible selected key, Q head), i.e. only each query's own
support.  `roofline` is for the dominant kernel (the union attention): the same
useful flops over its mean duration in the timed steps, against the 2.5 PFLOP/s
dense bf16 peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "complete-call latency (search+attn) & useful TFLOP/s, 64K prefill FP8 KV"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_64k")
    ap.add_argument("--no-arms", action="store_true", help="skip the identity / g=1 comparison arms")
    ap.add_argument("--only-arm", choices=["selector", "dense", "fp8qp"], default=None,
                    help="run only this comparison arm (for profiling it)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle sample time")
    ap.add_argument("--gen-workers", type=int, default=16,
                    help="processes for input generation (0: in-process, e.g. under a profiler)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the complete call over W in {32..1024} x g in {4, 8, 16} "
                         "(regrouped, and identity grouping at each g)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after the timed region, one plain 1 GiB device-to-device copy "
                         "(reference dispatch for scaling HBM byte counters)")
    return ap.parse_args()


def union_stats(sel: np.ndarray, ids: np.ndarray, g: int, N: int):
    """Per-group union sizes (pages) from the selections and the query IDs (host, numpy)."""
    H, T, S = sel.shape
    Ti = ids.shape[1]                    # ID entries per head (T, or a subset of each group)
    ng = (Ti + g - 1) // g
    pad = ng * g - Ti
    idp = np.concatenate([ids, np.full((H, pad), -1, ids.dtype)], axis=1) if pad else ids
    rows = np.where(idp[..., None] >= 0, np.take_along_axis(sel, np.clip(idp, 0, T - 1)[..., None], axis=1), -1)
    rows = rows.reshape(H, ng, g * S)
    rows = np.where((rows >= 0) & (rows < N), rows, -1)
    s = np.sort(rows, axis=2)
    distinct = s >= 0
    distinct[:, :, 1:] &= s[:, :, 1:] != s[:, :, :-1]
    return distinct.sum(axis=2)          # [H][ng]


def tile_units(sel: np.ndarray, ids: np.ndarray, g: int, G: int, N: int) -> int:
    """(32-row tile, page) units the attention computes: a group of g * G rows is cut into
    tiles of 32 rows (slot * G + head), and each tile walks the union of the pages its own
    slots selected."""
    n_rt = (g * G + 31) // 32
    if n_rt == 1:
        return int(union_stats(sel, ids, g, N).sum())
    H, T, S = sel.shape
    ng = (T + g - 1) // g
    pad = ng * g - T
    idp = np.concatenate([ids, np.full((H, pad), -1, ids.dtype)], axis=1) if pad else ids
    idp = idp.reshape(H, ng, g)
    total = 0
    for rt in range(n_rt):
        s_lo, s_hi = (32 * rt) // G, min(g - 1, (32 * rt + 31) // G)
        if s_lo > s_hi:
            continue
        sub = idp[:, :, s_lo:s_hi + 1].reshape(H, -1)
        total += int(union_stats(sel, sub, s_hi - s_lo + 1, N).sum())
    return total


def pair_entries(sel: np.ndarray, pairs, N: int) -> float:
    """Mean (query, page pair) entries per (KV head, query): adjacent pairs (2k, 2k+1) when
    `pairs` is None, else the int32 [H_kv][N][2] pair table."""
    H, T, S = sel.shape
    valid = (sel >= 0) & (sel < N)
    tot = 0
    for h in range(H):
        if pairs is None:
            pid = np.arange(N) // 2
        else:
            pid = np.full(N, -1, dtype=np.int64)
            for pos in (0, 1):
                col = pairs[h, :, pos]
                ok = col >= 0
                pid[col[ok]] = np.nonzero(ok)[0]
        k = np.where(valid[h], pid[np.clip(sel[h], 0, N - 1)], -1)
        k = np.sort(k, axis=1)
        distinct = k >= 0
        distinct[:, 1:] &= k[:, 1:] != k[:, :-1]
        tot += int(distinct.sum())
    return tot / (H * T)


KERNEL_FILES = ("query_union_paged_amd/csrc/union_attn.hip", "query_union_paged_amd/csrc/attn_common.h",
                "query_union_paged_amd/csrc/pw_internal.h", "query_union_paged_amd/build.py")


def kernel_hash() -> str:
    """Hash of the attention kernel's source, its shared header and the build flags."""
    h = hashlib.sha256()
    for f in KERNEL_FILES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """DRAM bytes of one union_attn_kernel launch, from the rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes stored under profiles/, each scaled by what the same counter reads for a plain
    1 GiB copy; None unless taken on this kernel source and build flags."""
    path = os.path.join(ROOT, "profiles", "union_attn_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    per = rec.get("workloads", {}).get(workload)
    if per is not None:
        return per.get("dram_bytes_per_launch")
    return rec.get("dram_bytes_per_launch") if rec.get("workload") == workload else None


def cpu_baseline(inp, wl, seconds: float):
    """The fp64 oracle on a bounded sample of the same workload (host cores)."""
    from oracle.attention import Problem, attention_pairs, attention_pairs_parallel
    from oracle.greedy import group_ids
    from query_union_paged_amd import synth
    workers = len(os.sched_getaffinity(0))
    pb = Problem(inp["q_bits"], inp["k_codes"], inp["v_codes"], inp["scales"], inp["sel_pages"])
    rng = np.random.default_rng(0)

    def sample(n):
        t = np.sort(rng.choice(wl.T, size=n, replace=False))
        return [(h, int(x)) for h in range(wl.H_kv) for x in t]
    # calibrate in-process (no pool start-up in the estimate), then size the sample
    from threadpoolctl import threadpool_limits
    cal = sample(4)
    with threadpool_limits(limits=1):
        t0 = time.time()
        attention_pairs(pb, cal)
        per_pair = (time.time() - t0) / len(cal)
    n = int(max(16, min(wl.T, seconds * workers / max(per_pair, 1e-6) / wl.H_kv)))
    for _ in range(2):          # resize once if the pool ran far from the target time
        pairs = sample(n)
        t0 = time.time()
        attention_pairs_parallel(pb, pairs, workers=workers)
        dt = time.time() - t0
        if dt >= 0.5 * seconds or n >= wl.T:
            break
        n = int(min(wl.T, n * seconds / max(dt, 1e-3)))
    sel = inp["sel_pages"]
    flops = 0.0
    for h, t in pairs:
        row = sel[h, t]
        u = np.unique(row[(row >= 0) & (row < wl.N)]).astype(np.int64)
        flops += float(np.clip(t - u * wl.P + 1, 0, wl.P).sum()) * wl.G * 4 * wl.D
    # the CPU greedy search on a sample of windows
    nwin = max(1, min(32, wl.T // wl.W))
    t1 = time.time()
    group_ids(sel, wl.N, wl.W, wl.g, workers=workers,
              windows={h: list(range(0, nwin * wl.W, wl.W)) for h in range(wl.H_kv)})
    gdt = time.time() - t1
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
        "sample": f"{len(pairs)} (KV head, query) rows ({n} stratified queries x {wl.H_kv} heads), "
                  f"fp64 numpy, {dt:.1f} s; full-job estimate {dt * wl.T / n:.0f} s",
        "greedy_windows_per_s": nwin * wl.H_kv / gdt,
        "greedy_full_estimate_s": gdt * (wl.T // wl.W) / nwin,
        "cpu_model": cpu_model(),
    }


def sweep(pw, torch, wl, inp, dev, shp, O, ws, reps: int = 5):
    """Complete-call cost over the window W and group size g (regrouped and identity)."""
    stream = torch.cuda.current_stream()
    ident = torch.arange(wl.T, dtype=torch.int32, device="cuda").repeat(wl.H_kv, 1).contiguous()
    ids = torch.empty_like(ident)

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def attn(g, idv):
        return lambda: pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"],
                                             dev["scales"], dev["sel_pages"], idv, g, O=O,
                                             workspace=ws)
    rows = []
    for g in (4, 8, 16):
        if g * wl.G > 64 or g * wl.S > 1024:
            continue
        a_id = timed(attn(g, ident))
        u_id = union_stats(inp["sel_pages"], ident.cpu().numpy(), g, wl.N)
        rows.append({"W": None, "g": g, "grouping": "identity", "search_ms": 0.0,
                     "attention_ms": a_id, "call_ms": a_id, "union_pages_mean": float(u_id.mean())})
        for W in (32, 64, 128, 256, 512, 1024):
            if W < g:
                continue
            s_ms = timed(lambda: pw.pw_group(shp, dev["sel_pages"], W, g, query_ids=ids))
            a_ms = timed(attn(g, ids))
            u = union_stats(inp["sel_pages"], ids.cpu().numpy(), g, wl.N)
            rows.append({"W": W, "g": g, "grouping": "regrouped", "search_ms": s_ms,
                         "attention_ms": a_ms, "call_ms": s_ms + a_ms,
                         "union_pages_mean": float(u.mean()), "vs_identity": a_id / (s_ms + a_ms)})
            log(f"[sweep] {wl.name} W={W} g={g}: search {s_ms:.3f} ms, attention {a_ms:.3f} ms, "
                f"union {u.mean():.1f} pages, identity {a_id:.3f} ms")
    return rows


def head_pipeline_arm(pw, torch, wl, dev, shp, O, ws, reps: int = 10):
    """The complete call with the search of later KV heads overlapping the attention of
    earlier ones (pw_group per head chunk on a second stream, pw_union_attention_heads per
    chunk on the caller's stream after its search), for chunks of 1, 2 and 4 heads."""
    stream = torch.cuda.current_stream()
    ids = torch.empty((wl.H_kv, wl.T), dtype=torch.int32, device="cuda")
    out = {}
    for chunk in (1, 2, 4):
        if wl.H_kv % chunk:
            continue
        run = pw.HeadPipeline(shp, chunk)
        call = lambda: run(dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                           dev["sel_pages"], wl.W, wl.g, ids, O, ws)
        for _ in range(2):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        out[f"chunk{chunk}_ms"] = a.elapsed_time(b) / reps
        log(f"[bench] head pipeline, {chunk} KV heads per chunk: {out[f'chunk{chunk}_ms']:.3f} ms")
    return out


def dense_arms(pw, torch, wl, inp, dev, shp, O, calls, cold_ms, F_u):
    """The direct KV-page union (design-study comparison), with adjacent pairs and with affinity
    pairs from the device's greedy co-selection matching (cold calls)."""
    q, k, v, sc, sel = dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"], dev["sel_pages"]
    arms = {}
    dws = torch.empty(pw.pw_dense_union_ref_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    dense = lambda: pw.pw_dense_union_ref(shp, q, k, v, sc, sel, O=O, workspace=dws)
    ms = cold_ms([dense], n=2)
    arms["direct_page_union"] = {"ms": ms, "useful_TFLOPs": F_u / (ms * 1e-3) / 1e12,
                                 "workspace_GiB": dws.numel() / 2 ** 30,
                                 "entries_per_query": pair_entries(inp["sel_pages"], None, wl.N)}
    # the same with affinity pairs (greedy co-selection matching on the device)
    pws = torch.empty(pw.pw_page_pairs_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    prs = pw.pw_page_pairs(shp, sel, workspace=pws)
    pairing = lambda: pw.pw_page_pairs(shp, sel, pairs=prs, workspace=pws)
    dense_p = lambda: pw.pw_dense_union_ref(shp, q, k, v, sc, sel, O=O, workspace=dws, pairs=prs)
    calls.run([pairing, dense_p], 1, cold=False)
    t = np.median(calls.run([pairing, dense_p], 2, cold=True), axis=0)
    arms["direct_page_union_affinity"] = {
        "pairing_ms": float(t[0]), "union_ms": float(t[1]), "ms": float(t.sum()),
        "useful_TFLOPs": F_u / (float(t.sum()) * 1e-3) / 1e12,
        "entries_per_query": pair_entries(inp["sel_pages"], prs.cpu().numpy(), wl.N)}
    log(f"[bench] direct page union: adjacent {ms:.2f} ms, affinity {t[0]:.2f} + {t[1]:.2f} ms")
    del dws, pws
    return arms


def ordered_stages(pw, torch, wl, shp, q, k, v, sc, sel, ws, O):
    """The complete call with each KV head's groups run in the order pw_group_ordered emits
    (blocks of the groups one XCD runs at once, each by ascending union size):
    pw_group_ordered + pw_tile_kv + pw_union_attention_tiled_ordered."""
    import ctypes
    ids = torch.empty((wl.H_kv, wl.T), dtype=torch.int32, device="cuda")
    order = torch.empty((wl.H_kv, -(-wl.T // wl.g)), dtype=torch.int32, device="cuda")
    gws = torch.empty(max(1, int(pw._lib.pw_group_ordered_workspace_bytes(
        ctypes.byref(shp), wl.W, wl.g))), dtype=torch.uint8, device="cuda")
    return [lambda: pw.pw_group_ordered(shp, sel, wl.W, wl.g, query_ids=ids, group_order=order,
                                        workspace=gws),
            lambda: pw.pw_tile_kv(shp, k, v, sc, workspace=ws),
            lambda: pw.pw_union_attention_tiled(shp, q, sel, ids, wl.g, ws, O=O,
                                                group_order=order)]


def selector_arm(pw, torch, wl, dev, shp, O, ws, ident, cold_ms):
    """The synthetic GPU selector (sink + 2 local pages + top pages by block key sums) and the
    complete call on its selections, regrouped (in the search's group order, and in the order
    pw_group_ordered emits) and with identity grouping (cold calls)."""
    sws = torch.empty(pw.pw_select_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    sel = torch.empty_like(dev["sel_pages"])
    ids = torch.empty((wl.H_kv, wl.T), dtype=torch.int32, device="cuda")
    q, k, v, sc = dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"]
    select = lambda: pw.pw_select(shp, q, k, sc, 2, sel_pages=sel, workspace=sws)
    search = lambda: pw.pw_group(shp, sel, wl.W, wl.g, query_ids=ids)
    tile = lambda: pw.pw_tile_kv(shp, k, v, sc, workspace=ws)
    attn = lambda idv: (lambda: pw.pw_union_attention_tiled(shp, q, sel, idv, wl.g, ws, O=O))
    sel_ms = cold_ms([select])
    select()
    ordered = ordered_stages(pw, torch, wl, shp, q, k, v, sc, sel, ws, O)
    call_ms, ordered_ms, ident_ms = [], [], []
    for _ in range(2):                   # alternated, so that drift hits every arm alike
        call_ms.append(cold_ms([search, tile, attn(ids)], n=4))
        ordered_ms.append(cold_ms(ordered, n=4))
        ident_ms.append(cold_ms([tile, attn(ident)], n=4))
    call_ms, ordered_ms, ident_ms = (float(np.median(x)) for x in (call_ms, ordered_ms, ident_ms))
    sel_np = sel.cpu().numpy()
    u = union_stats(sel_np, ids.cpu().numpy(), wl.g, wl.N)
    ui = union_stats(sel_np, ident.cpu().numpy(), wl.g, wl.N)
    del sws
    # call_ms / regroup_gain_vs_identity: the same complete call as the headline (with the
    # group order); search_order_*: pw_group + pw_union_attention_tiled in the search's order
    return {"select_ms": sel_ms, "call_ms": ordered_ms, "search_order_call_ms": call_ms,
            "identity_call_ms": ident_ms,
            "regroup_gain_vs_identity": ident_ms / ordered_ms,
            "search_order_regroup_gain_vs_identity": ident_ms / call_ms,
            "union_pages_mean": float(u.mean()), "union_pages_std": float(u.std()),
            "identity_union_pages_mean": float(ui.mean()), "n_local": 2}


def fp8qp_arm(pw, torch, wl, shp, q, k, v, sc, sel, ws, calls, F_u, O_exact, n: int = 10):
    """The complete call with the lower-precision attention (Q and P in e4m3fn,
    pw_union_attention_tiled_fp8qp) in the order pw_group_ordered emits, cold, and how far its
    output lies from the exact path's output on the same inputs."""
    import ctypes
    ids = torch.empty((wl.H_kv, wl.T), dtype=torch.int32, device="cuda")
    order = torch.empty((wl.H_kv, -(-wl.T // wl.g)), dtype=torch.int32, device="cuda")
    gws = torch.empty(max(1, int(pw._lib.pw_group_ordered_workspace_bytes(
        ctypes.byref(shp), wl.W, wl.g))), dtype=torch.uint8, device="cuda")
    O8 = torch.empty_like(O_exact)
    stages = [lambda: pw.pw_group_ordered(shp, sel, wl.W, wl.g, query_ids=ids, group_order=order,
                                          workspace=gws),
              lambda: pw.pw_tile_kv(shp, k, v, sc, workspace=ws),
              lambda: pw.pw_union_attention_tiled_fp8qp(shp, q, sel, ids, wl.g, ws, O=O8,
                                                        group_order=order)]
    calls.run(stages, 1, cold=False)
    t = calls.run(stages, n, cold=True)
    call_ms = float(np.median(t.sum(axis=1)))
    kern_ms = float(t[:, 2].mean())
    d = (O8.float() - O_exact.float()).abs()
    log(f"[bench] fp8 Q and P: call {call_ms:.3f} ms, attention {kern_ms:.3f} ms")
    return {"ms": call_ms, "useful_TFLOPs": F_u / (call_ms * 1e-3) / 1e12,
            "attention_ms": kern_ms, "attention_frac": F_u / (kern_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "vs_exact_path_output": {"max_abs": float(d.max()), "mean_abs": float(d.mean())}}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Calls:
    """Cold and warm timing of device calls on one stream.  A cold call is preceded by a
    1 GiB write (outside its events) that evicts the MALL and the L2."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def run(self, stages, n: int, cold: bool):
        """stages: list of callables run back to back; returns [n][len(stages)] ms."""
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(n)]
        for row in ev:
            if cold:
                self.flush.fill_(1.0)
            row[0].record(self.stream)
            for fn, e in zip(stages, row[1:]):
                fn()
                e.record(self.stream)
        torch.cuda.synchronize()
        return np.array([[row[i].elapsed_time(row[i + 1]) for i in range(len(stages))]
                         for row in ev])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no communication between GPUs).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from query_union_paged_amd import pageweaver as pw
    from query_union_paged_amd import synth

    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    inp = synth.make_qkv(wl)
    inp["sel_pages"] = synth.make_selection(
        wl, workers=min(args.gen_workers, len(os.sched_getaffinity(0))))
    log(f"[bench] inputs {wl.name} generated in {time.time() - t0:.1f}s")
    dev = pw.to_device(inp)
    shp = pw.shape(*wl.shape_tuple())
    F_u = synth.useful_flops(inp["sel_pages"], wl)

    ids = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    ws = torch.empty(pw.pw_union_attention_workspace_bytes(shp, wl.g), dtype=torch.uint8,
                     device="cuda")
    O = torch.empty((wl.T, wl.H_q, wl.D), dtype=torch.bfloat16, device="cuda")
    q, k, v, sc, sel = dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"], dev["sel_pages"]

    def search(sel_=sel, ids_=ids, W=wl.W, g=wl.g):
        return lambda: pw.pw_group(shp, sel_, W, g, query_ids=ids_)

    tile = lambda: pw.pw_tile_kv(shp, k, v, sc, workspace=ws)

    def attend(ids_=ids, g=wl.g, sel_=sel):
        return lambda: pw.pw_union_attention_tiled(shp, q, sel_, ids_, g, ws, O=O)

    order = torch.empty((wl.H_kv, -(-wl.T // wl.g)), dtype=torch.int32, device="cuda")
    gws = torch.empty(max(1, pw.pw_group_ordered_workspace_bytes(shp, wl.W, wl.g)),
                      dtype=torch.uint8, device="cuda")
    search_ordered = lambda: pw.pw_group_ordered(shp, sel, wl.W, wl.g, query_ids=ids,
                                                 group_order=order, workspace=gws)
    attend_ordered = lambda: pw.pw_union_attention_tiled(shp, q, sel, ids, wl.g, ws, O=O,
                                                         group_order=order)
    stages = [search_ordered, tile, attend_ordered]
    calls = Calls(torch)
    calls.run(stages, args.warmup, cold=False)           # untimed warm-up
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    cold = calls.run(stages, args.steps, cold=True)       # the K timed steps (synchronised)
    wall = time.perf_counter() - t_start
    warm = calls.run(stages, args.steps, cold=False)
    call_cold = cold.sum(axis=1)
    call_warm = warm.sum(axis=1)
    ms_per_step = float(np.median(call_cold))
    value = F_u / (ms_per_step * 1e-3) / 1e12

    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                       # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    # roofline of the dominant kernel (union_attn_kernel, launched by
    # pw_union_attention_tiled_ordered)
    ids_np = ids.cpu().numpy()
    usz = union_stats(inp["sel_pages"], ids_np, wl.g, wl.N)
    n_pages_total = tile_units(inp["sel_pages"], ids_np, wl.g, wl.G, wl.N)   # (tile, page) units
    rows = wl.g * wl.G
    comp_unit = 4 * 32 * wl.P * wl.D                # MFMA flops per (32-row tile, page)
    comp_flops = n_pages_total * comp_unit
    attn_s = float(cold[:, 2].mean()) * 1e-3
    achieved = F_u / attn_s / 1e12
    tiled_bytes = pw.pw_union_attention_workspace_bytes(shp, wl.g)
    compulsory = (2 * wl.T * wl.H_q * wl.D * 2 + inp["sel_pages"].nbytes + ids_np.nbytes
                  + tiled_bytes)                   # Q, O, selections, IDs, tiled K/V read once
    traffic = recorded_traffic(wl.name)
    roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS, "traffic": traffic,
            "kernel": "union_attn_kernel (pw_union_attention_tiled_ordered), mean of the timed cold steps",
            "flops_per_unit": 4 * wl.D, "unit_def": "(visible selected key, Q head) pair",
            "units_per_launch": F_u / (4 * wl.D), "kernel_ms": attn_s * 1e3,
            "complete_call": {"achieved": value, "frac": value / BF16_MFMA_PEAK_TFLOPS,
                              "ms": ms_per_step},
            "computed_work": {"flops": comp_flops, "per_tile_page": comp_unit,
                              "tile_pages": n_pages_total,
                              "achieved": comp_flops / attn_s / 1e12,
                              "frac": comp_flops / attn_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                              "useful_over_computed": F_u / comp_flops},
            "dram": {"compulsory_bytes": compulsory,
                     "measured_bytes": traffic,
                     "measured_over_compulsory": (traffic / compulsory) if traffic else None,
                     "measured_GBs": (traffic / attn_s / 1e9) if traffic else None,
                     "peak_GBs": HBM_PEAK_GBS}}

    def cold_ms(stages_, n=5):
        calls.run(stages_, 1, cold=False)
        return float(np.median(calls.run(stages_, n, cold=True).sum(axis=1)))

    arms = {}
    ident = torch.arange(wl.T, dtype=torch.int32, device="cuda").repeat(wl.H_kv, 1).contiguous()
    if args.only_arm == "selector":
        arms["selector"] = selector_arm(pw, torch, wl, dev, shp, O, ws, ident, cold_ms)
    elif args.only_arm == "dense":
        arms.update(dense_arms(pw, torch, wl, inp, dev, shp, O, calls, cold_ms, F_u))
    elif args.only_arm == "fp8qp":
        arms["fp8qp"] = fp8qp_arm(pw, torch, wl, shp, q, k, v, sc, sel, ws, calls, F_u, O)
    elif not args.no_arms:
        for name, g_arm in [("identity_union8", wl.g), ("per_query_g1", 1)]:
            ms = cold_ms([tile, attend(ident, g_arm)], n=5 if g_arm == 1 else 10)
            us = union_stats(inp["sel_pages"], ident.cpu().numpy(), g_arm, wl.N)
            arms[name] = {"ms": ms, "useful_TFLOPs": F_u / (ms * 1e-3) / 1e12,
                          "union_pages_mean": float(us.mean()), "union_pages_total": int(us.sum())}
        arms["regroup_gain_vs_identity"] = arms["identity_union8"]["ms"] / ms_per_step
        ms = cold_ms([search(), tile, attend()], n=10)
        arms["regrouped_search_order"] = {"ms": ms, "useful_TFLOPs": F_u / (ms * 1e-3) / 1e12}
        arms.update(dense_arms(pw, torch, wl, inp, dev, shp, O, calls, cold_ms, F_u))
        arms["selector"] = selector_arm(pw, torch, wl, dev, shp, O, ws, ident, cold_ms)
        arms["head_pipeline"] = head_pipeline_arm(pw, torch, wl, dev, shp, O, ws)
        stages[-1]()                     # O = the exact path's output again
        arms["fp8qp"] = fp8qp_arm(pw, torch, wl, shp, q, k, v, sc, sel, ws, calls, F_u, O)

    swp = sweep(pw, torch, wl, inp, dev, shp, O, ws) if args.sweep else None

    cpu = None
    if not args.no_cpu:
        t0 = time.time()
        cpu = cpu_baseline(inp, wl, args.cpu_seconds)
        log(f"[bench] cpu baseline {time.time() - t0:.1f}s")

    def stats(a):
        return {"median": float(np.median(a)), "p90": float(np.percentile(a, 90)),
                "mean": float(np.mean(a))}

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3/bf16",
        "data": "synthetic (seeded captures, Q/K/V ~ N(0,1), e4m3fn KV with per-page scales)",
        "config": {"workload": wl.name, "tokens": wl.T, "H_q": wl.H_q, "H_kv": wl.H_kv,
                   "head_dim": wl.D, "page": wl.P, "selected_pages": wl.S, "W": wl.W, "g": wl.g,
                   "kv": "fp8_e4m3fn", "grouping": "regrouped, group order of pw_group_ordered",
                   "timing": "cold (MALL+L2 flushed)"},
        "latency_ms": {"complete_call_cold": stats(call_cold), "complete_call_warm": stats(call_warm),
                       "search_cold": stats(cold[:, 0]), "tile_kv_cold": stats(cold[:, 1]),
                       "attention_cold": stats(cold[:, 2]), "search_warm": stats(warm[:, 0]),
                       "tile_kv_warm": stats(warm[:, 1]), "attention_warm": stats(warm[:, 2]),
                       "timed_region_wall_s": wall},
        "warm_value": F_u / (float(np.median(call_warm)) * 1e-3) / 1e12,
        "useful_flops": F_u,
        "union": {"pages_mean": float(usz.mean()), "pages_max": int(usz.max()),
                  "efficiency_useful_over_computed": F_u / comp_flops},
        "roofline": roof, "arms": arms, "cpu_baseline": cpu,
        **({"sweep": swp} if swp is not None else {}),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
