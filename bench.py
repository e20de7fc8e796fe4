"""Complete-call benchmark of query-union sparse-attention prefill on one MI355X.

One step = one complete call on resident inputs: the grouping search
(pw_group) followed by the union attention (pw_union_attention), both on the
same stream.  Default workload: 64K-token prefill of a Llama-3-8B-like layer
(32 Q / 8 KV heads, d = 128, page 64, 64 selected pages per (query, KV head),
Zipf(1.1) community draws, W = 256, g = 8), FP8 e4m3fn KV, bf16 Q and O.

Prints one JSON line (rank 0).  `value` is useful TFLOP/s: 4*D flops per
(visible selected key, Q head), i.e. only each query's own support.
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
    ap.add_argument("--only-arm", choices=["selector"], default=None,
                    help="run only this comparison arm (for profiling it)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU oracle sample time")
    ap.add_argument("--cold", type=int, default=5, help="cold-cache runs (MALL/L2 flushed)")
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
    ng = (T + g - 1) // g
    pad = ng * g - T
    idp = np.concatenate([ids, np.full((H, pad), -1, ids.dtype)], axis=1) if pad else ids
    rows = np.where(idp[..., None] >= 0, np.take_along_axis(sel, np.clip(idp, 0, T - 1)[..., None], axis=1), -1)
    rows = rows.reshape(H, ng, g * S)
    rows = np.where((rows >= 0) & (rows < N), rows, -1)
    s = np.sort(rows, axis=2)
    distinct = s >= 0
    distinct[:, :, 1:] &= s[:, :, 1:] != s[:, :, :-1]
    return distinct.sum(axis=2)          # [H][ng]


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


def kernel_hash() -> str:
    src = os.path.join(ROOT, "query_union_paged_amd", "csrc", "union_attn.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def recorded_traffic():
    """HBM bytes of one pw_union_attention call (re-tiling + attention kernels), from the
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes stored under profiles/, each scaled by what the
    same counter reads for a plain 1 GiB copy; None unless taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "union_attn_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_call")


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


def selector_arm(pw, torch, wl, dev, shp, O, ws, reps: int = 5):
    """The synthetic GPU selector (sink + 2 local pages + top pages by block key sums) and the
    complete call on its selections, regrouped and with identity grouping."""
    stream = torch.cuda.current_stream()
    sws = torch.empty(pw.pw_select_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
    sel = torch.empty_like(dev["sel_pages"])
    ids = torch.empty((wl.H_kv, wl.T), dtype=torch.int32, device="cuda")
    ident = torch.arange(wl.T, dtype=torch.int32, device="cuda").repeat(wl.H_kv, 1).contiguous()

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def attn(idv):
        return lambda: pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"],
                                             dev["scales"], sel, idv, wl.g, O=O, workspace=ws)
    sel_ms = timed(lambda: pw.pw_select(shp, dev["q_bits"], dev["k_codes"], dev["scales"], 2,
                                        sel_pages=sel, workspace=sws))
    search_ms = timed(lambda: pw.pw_group(shp, sel, wl.W, wl.g, query_ids=ids))
    attn_ms = timed(attn(ids))
    ident_ms = timed(attn(ident))
    sel_np = sel.cpu().numpy()
    u = union_stats(sel_np, ids.cpu().numpy(), wl.g, wl.N)
    ui = union_stats(sel_np, ident.cpu().numpy(), wl.g, wl.N)
    del sws
    return {"select_ms": sel_ms, "search_ms": search_ms, "attention_ms": attn_ms,
            "call_ms": search_ms + attn_ms, "identity_attention_ms": ident_ms,
            "regroup_gain_vs_identity": ident_ms / (search_ms + attn_ms),
            "union_pages_mean": float(u.mean()), "identity_union_pages_mean": float(ui.mean()),
            "n_local": 2}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no communication; see the design notes).",
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
    stream = torch.cuda.current_stream()
    F_u = synth.useful_flops(inp["sel_pages"], wl)

    ids = pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g)
    ws = torch.empty(pw.pw_union_attention_workspace_bytes(shp, wl.g), dtype=torch.uint8,
                     device="cuda")
    O = pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, wl.g, workspace=ws)
    torch.cuda.synchronize()

    def step():
        pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g, query_ids=ids)
        pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, wl.g, O=O, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        pw.pw_group(shp, dev["sel_pages"], wl.W, wl.g, query_ids=ids)
        e1.record(stream)
        pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], ids, wl.g, O=O, workspace=ws)
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    search_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    attn_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    ms_per_step = wall * 1e3 / args.steps
    value = F_u / (ms_per_step * 1e-3) / 1e12

    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)                       # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst

    # cold runs: a 1 GiB write between runs evicts MALL and L2
    cold = []
    if args.cold > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        for _ in range(args.cold):
            flush.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        del flush

    # union accounting for the roofline (host-side, from the IDs the search returned)
    ids_np = ids.cpu().numpy()
    usz = union_stats(inp["sel_pages"], ids_np, wl.g, wl.N)
    n_units = int(usz.sum())                       # (group, union page) pairs per launch
    page_bytes = 2 * wl.P * wl.D                   # K + V e4m3fn bytes of one (page, KV head)
    qo_bytes = 2 * wl.T * wl.H_q * wl.D * 2
    meta_bytes = inp["sel_pages"].nbytes * 2 + ids_np.nbytes + inp["scales"].nbytes
    alg_bytes = n_units * page_bytes + qo_bytes + meta_bytes
    rows = wl.g * wl.G
    flop_unit = 4 * ((rows + 31) // 32 * 32) * wl.P * wl.D   # QK^T + PV MFMA work per (group, page)
    comp_flops = n_units * flop_unit
    attn_avg_s = float(attn_ms.mean()) * 1e-3
    mfma_tflops = comp_flops / attn_avg_s / 1e12
    gbs = alg_bytes / attn_avg_s / 1e9
    traffic = recorded_traffic()
    roof = {"bound": "mfma", "achieved": mfma_tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": mfma_tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": traffic,
            "kernel": "pw_union_attention call (tile_kv_kernel + union_attn_kernel)",
            "flops_per_unit": flop_unit,
            "units_per_launch": n_units,
            "hbm_definition": {"algorithmic_bytes": alg_bytes, "achieved_GBs": gbs,
                               "peak_GBs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS}}

    arms = {}
    if args.only_arm == "selector":
        arms["selector"] = selector_arm(pw, torch, wl, dev, shp, O, ws)
    elif not args.no_arms:
        ident = torch.arange(wl.T, dtype=torch.int32, device="cuda").repeat(wl.H_kv, 1).contiguous()
        for name, g_arm, ids_arm in [("identity_union8", wl.g, ident), ("per_query_g1", 1, ident)]:
            n = 5 if g_arm == 1 else 10
            for _ in range(2):
                pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"],
                                      dev["scales"], dev["sel_pages"], ids_arm, g_arm, O=O,
                                      workspace=ws)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                pw.pw_union_attention(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"],
                                      dev["scales"], dev["sel_pages"], ids_arm, g_arm, O=O,
                                      workspace=ws)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / n
            us = union_stats(inp["sel_pages"], ids_arm.cpu().numpy(), g_arm, wl.N)
            arms[name] = {"ms": ms, "useful_TFLOPs": F_u / (ms * 1e-3) / 1e12,
                          "union_pages_mean": float(us.mean()), "union_pages_total": int(us.sum())}
        arms["regroup_gain_vs_identity"] = arms["identity_union8"]["ms"] / ms_per_step
        # the direct KV-page union (design-study comparison)
        dws = torch.empty(pw.pw_dense_union_ref_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
        pw.pw_dense_union_ref(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], O=O, workspace=dws)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(2):
            pw.pw_dense_union_ref(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                                  dev["sel_pages"], O=O, workspace=dws)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 2
        arms["direct_page_union"] = {"ms": ms, "useful_TFLOPs": F_u / (ms * 1e-3) / 1e12,
                                     "workspace_GiB": dws.numel() / 2 ** 30,
                                     "entries_per_query": pair_entries(inp["sel_pages"], None, wl.N)}
        # the same with affinity pairs (greedy co-selection matching on the device)
        pws = torch.empty(pw.pw_page_pairs_workspace_bytes(shp), dtype=torch.uint8, device="cuda")
        prs = pw.pw_page_pairs(shp, dev["sel_pages"], workspace=pws)
        pw.pw_dense_union_ref(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                              dev["sel_pages"], O=O, workspace=dws, pairs=prs)
        t = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t[0].record(stream)
        for _ in range(2):
            pw.pw_page_pairs(shp, dev["sel_pages"], pairs=prs, workspace=pws)
        t[1].record(stream)
        for _ in range(2):
            pw.pw_dense_union_ref(shp, dev["q_bits"], dev["k_codes"], dev["v_codes"], dev["scales"],
                                  dev["sel_pages"], O=O, workspace=dws, pairs=prs)
        t[2].record(stream)
        torch.cuda.synchronize()
        pair_ms, du_ms = t[0].elapsed_time(t[1]) / 2, t[1].elapsed_time(t[2]) / 2
        arms["direct_page_union_affinity"] = {
            "pairing_ms": pair_ms, "union_ms": du_ms, "ms": pair_ms + du_ms,
            "useful_TFLOPs": F_u / ((pair_ms + du_ms) * 1e-3) / 1e12,
            "entries_per_query": pair_entries(inp["sel_pages"], prs.cpu().numpy(), wl.N)}
        log(f"[bench] direct page union: adjacent {ms:.2f} ms, affinity {pair_ms:.2f} + {du_ms:.2f} ms")
        del dws, pws
        arms["selector"] = selector_arm(pw, torch, wl, dev, shp, O, ws)
        arms["head_pipeline"] = head_pipeline_arm(pw, torch, wl, dev, shp, O, ws)

    swp = sweep(pw, torch, wl, inp, dev, shp, O, ws) if args.sweep else None

    cpu = None
    if not args.no_cpu:
        t0 = time.time()
        cpu = cpu_baseline(inp, wl, args.cpu_seconds)
        log(f"[bench] cpu baseline {time.time() - t0:.1f}s")

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3/bf16",
        "data": "synthetic (seeded captures, Q/K/V ~ N(0,1), e4m3fn KV with per-page scales)",
        "config": {"workload": wl.name, "tokens": wl.T, "H_q": wl.H_q, "H_kv": wl.H_kv,
                   "head_dim": wl.D, "page": wl.P, "selected_pages": wl.S, "W": wl.W, "g": wl.g,
                   "kv": "fp8_e4m3fn", "grouping": "regrouped"},
        "latency_ms": {"complete_call": ms_per_step, "search_mean": float(search_ms.mean()),
                       "attention_mean": float(attn_ms.mean()),
                       "attention_median": float(np.median(attn_ms)),
                       "attention_p90": float(np.percentile(attn_ms, 90)),
                       "complete_call_cold_median": float(np.median(cold)) if cold else None},
        "useful_flops": F_u,
        "union": {"pages_mean": float(usz.mean()), "pages_max": int(usz.max()),
                  "efficiency_useful_over_computed": F_u / comp_flops},
        "roofline": roof, "arms": arms, "cpu_baseline": cpu,
        **({"sweep": swp} if swp is not None else {}),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
