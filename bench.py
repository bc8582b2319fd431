"""Benchmark: ADA paged decode on one MI355X.

One step = one full decode of the workload (`ada_decode`): the split-K pass
(angle-LUT staging, logits from codes, online softmax, value accumulation)
followed by the reduction pass, for every (sequence, query head), with the
packed cache already resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]

Reported value: kept KV token-heads scanned per second (a token-head is one
(token, KV head) entry of the cache; dropped tokens are absent from the
pages).  The roofline entry prices the split-K kernel's algorithmic bytes
(radius + codes + fp16 values per kept token-head, 12 bytes of metadata and
page-table per page, the queries) against MI355X's 8 TB/s HBM peak.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
# radius + codes + values per token-head (head dim 128): fp16 values (tiers
# 0-2) or V8 values, 4 scale bytes + 128 codes (tiers 3-5)
TIER_TOKEN_BYTES = {0: 386, 1: 322, 2: 298, 3: 262, 4: 198, 5: 174}
TIERS = range(6)
DENSE_TOKEN_BYTES = 512
METRIC = "ADA decode KV-tokens/sec and achieved HBM GB/s (% of peak) at 32k–128k ctx"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (about 30 ms at llama8b; shorter warm-ups measured 3%% slower steps)")
    ap.add_argument("--workload", default="llama8b", choices=["llama8b", "rdr128k", "ragged", "long256k", "tiny"])
    ap.add_argument("--chunk-pages", type=int, default=0)
    ap.add_argument("--utility", action="store_true",
                    help="time decode with per-token utility emission against plain decode")
    ap.add_argument("--append", action="store_true",
                    help="time the fused append + decode step against append then decode")
    ap.add_argument("--repack", type=float, default=0.0, metavar="FRAC",
                    help="time ada_repack of the packed cache to FRAC of its current bytes instead")
    ap.add_argument("--repack-mask", type=int, default=0,
                    help="RDR tier mask of the re-pack (0: T8, T4, T2; 56: the V8 tiers)")
    ap.add_argument("--setup", action="store_true",
                    help="time the setup path instead: ada_pack (exact encoding and page placement) of the "
                         "workload, and ada_rdr_assign of the rdr128k utilities")
    ap.add_argument("--v8", action="store_true",
                    help="store every kept token's values in V8 (tiers 3-5: the same keys, 8-bit values)")
    ap.add_argument("--queries", type=int, default=1,
                    help="queries per sequence (multi-query decode; Q * Hq/Hkv <= 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=100,
                    help="extra split-K launches each after 1 GiB of unrelated reads (cold caches), untimed in value")
    ap.add_argument("--others", default="rdr128k,ragged,long256k",
                    help="further workloads measured after the headline one, each reported in `workloads` "
                         "(comma-separated; empty for none)")
    return ap.parse_args()


def release(torch, settle_s=1.5):
    """Return freed device memory to the driver, then let the device settle
    before the next timed region.  For a while after several GB are
    released the driver works on that memory in the background: a decode
    timed right after freeing the ragged workload's 6.4 GB of input keys and
    values ran 3% slower (192.8 against 187.3 us after a one-second pause),
    and rdr128k alternated between 132.6 and 137.7 us."""
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    time.sleep(settle_s)


def kernel_source_hash():
    """Hash of the split-K kernel's sources with comments and blank lines
    removed (a comment edit does not change the kernel)."""
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_core.h", "ada_internal.h"):
        with open(os.path.join(ROOT, "compressed_kv_cache_ada_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per split-K launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"ada_decode_partials_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def build_workload(name, torch, ada, W):
    w = W.config(name)
    if w["tiers"] is None:   # RDR workload: the packer decides the tiers first
        cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"])
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        t = ada.rdr_assign(cfg, w["ctx_len"], torch.from_numpy(w["utility"]).cuda(), w["budget"], status)
        assert ada.read_status(status) == ada.OK
        w["tiers"] = t.cpu().numpy()
    return w


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding of the decode is described, not built)"}))
        sys.exit(2)
    import torch
    import compressed_kv_cache_ada_amd as ada
    import workloads as W

    torch.cuda.set_device(0)
    w = build_workload(args.workload, torch, ada, W)
    if args.v8:
        w["tiers"] = np.where(w["tiers"] >= 0, w["tiers"] + 3, -1).astype(np.int8)
    P, Hq, Hkv, B = w["P"], w["Hq"], w["Hkv"], w["B"]
    kept, pages_by_tier, max_row, n_pages, units = workload_shape(w, ada)

    cfg = ada.make_config(P, Hq, Hkv, decode_chunk_pages=args.chunk_pages, value_tiers=args.v8)
    if args.append:
        append_bench(args, w, ada, torch, cfg, kept, max_row, n_pages, units)
        return
    if args.repack > 0:
        repack_bench(args, w, ada, torch, cfg, kept, max_row, n_pages, units)
        return
    if args.utility:
        utility_bench(args, w, ada, torch, cfg, kept, max_row, n_pages, units)
        return
    if args.setup:
        setup_bench(args, w, ada, torch, W, cfg, kept, max_row, n_pages, units)
        return
    m = measure_decode(args, w, ada, torch, cfg, kept, max_row, n_pages, units, args.steps, args.cold_steps)
    Q = args.queries
    # copy probe: streaming ceiling of this machine (read + write bytes)
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        ada.probe_copy(src, dst, nb)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        ada.probe_copy(src, dst, nb)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # read ceiling: best of the streaming-read variants over 1 GiB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    read_gbps = {}
    for variant in range(6):   # 5: random 16 KB chunks per wavefront, the decode's pattern
        for _ in range(2):
            ada.probe_read(src, nb, variant, sink)
        e0.record()
        for _ in range(10):
            ada.probe_read(src, nb, variant, sink)
        e1.record()
        torch.cuda.synchronize()
        read_gbps[variant] = nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    release(torch)

    alg_bytes = m["alg_bytes"]
    achieved = alg_bytes / (m["kernel_ms"] * 1e-3) / 1e9
    traffic = measured_traffic(args.workload + ("_v8" if args.v8 else "")) if Q == 1 else None
    ms_step = m["ms_per_step"]
    value = m["kept"] / (ms_step * 1e-3)

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "KV token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128,
            "context": int(w["ctx_len"].max()), "page_size": P, "kept_token_heads": m["kept"],
            "kept_by_tier": [kept[t] for t in TIERS],        # tier ids 0-5: T8, T4, T2, T8V8, T4V8, T2V8
            "pages_by_tier": m["pages_by_tier"],
            "values": "V8" if args.v8 else "fp16",
            # footprint: every page is one arena block (key part, then values)
            "cache_arena_bytes": units * 16, "cache_arena_bytes_per_kept_token_head": units * 16 / m["kept"],
            "decode_chunk_pages": cfg.decode_chunk_pages, "queries_per_sequence": Q,
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
            "kernel": "decode_partials_kernel" if Q == 1 else "decode_partials_kernel + decode_reduce_kernel",
            "kernel_ms": m["kernel_ms"], "kernel_ms_event_per_launch": m["kernel_ms_event_mean"],
            "kernel_ms_event_median": m["kernel_ms_event_median"],
            "frac_of_read_probe": None,
            "reduce_kernel_ms": m["reduce_kernel_ms"],
            "algorithmic_bytes": alg_bytes,
        },
        # spread of the headline over the individually event-timed steps
        "value_p10": m["value_p10"], "value_p90": m["value_p90"],
        "ms_per_step_event_p10": m["ms_per_step_event_p10"], "ms_per_step_event_p90": m["ms_per_step_event_p90"],
        "graph_ms_per_step": m["graph_ms_per_step"],
        "ms_per_step_with_events": m["ms_per_step_with_events"],
        "step_hbm_gbps": m["step_hbm_gbps"],
        "context_tokens_per_s": m["context_tokens_per_s"],
        "cold_kernel_ms_median": m["cold_kernel_ms_median"],
        "cold_gbps": m["cold_gbps"],
        "copy_probe_gbps": copy_gbps,
        "read_probe_gbps": max(read_gbps[v] for v in range(4)),
        "read_probe_variants_gbps": read_gbps,
        # the ceiling of the decode's own access pattern (random 16 KB
        # chunks per wavefront, three work-groups per compute unit)
        "chunk_probe_gbps": read_gbps[5],
        "kernel_source_hash": kernel_source_hash(),
    }

    if Q > 1:
        result["query_token_heads_per_s"] = value * Q   # (query, kept token-head) pairs scored per second
    if not args.no_dense and Q == 1:
        result["dense_fp16_reference"] = dense_reference(w, ada, torch, cfg)
    if not args.no_cpu_baseline and Q == 1:
        result["cpu_baseline"] = cpu_baseline(w, m["kept"], max_row, n_pages, units)
    result["roofline"]["frac_of_read_probe"] = achieved / result["read_probe_gbps"]
    result["roofline"]["frac_of_chunk_probe"] = achieved / read_gbps[5]
    # the other workloads of the metric's context range, each timed the same way
    others = [x for x in args.others.split(",") if x and x != args.workload] if Q == 1 and not args.v8 else []
    if others:
        del w
        result["workloads"] = {}
        for name in others:
            result["workloads"][name] = other_workload(name, args, ada, torch, W, result["read_probe_gbps"],
                                                       read_gbps[5])
    print(json.dumps(result), flush=True)


def workload_shape(w, ada):
    """Kept token-heads and pages per tier, the longest row, pages and code
    units of a packed cache of the workload."""
    P, Hkv, B = w["P"], w["Hkv"], w["B"]
    tiers = w["tiers"]
    kept = {t: int((tiers == t).sum()) for t in TIERS}
    pages_by_tier = {t: 0 for t in TIERS}
    max_row = 0
    for b in range(B):
        for h in range(Hkv):
            rp = 0
            for t in TIERS:
                n = int((tiers[b, h] == t).sum())
                pages_by_tier[t] += -(-n // P)
                rp += -(-n // P)
            max_row = max(max_row, rp)
    n_pages = sum(pages_by_tier.values())
    units = sum(pages_by_tier[t] * ada.block_bytes(t, P) // 16 for t in TIERS)
    return kept, pages_by_tier, max_row, n_pages, units


def other_workload(name, args, ada, torch, W, read_probe_gbps, chunk_probe_gbps):
    """One further workload: decode timing as for the headline (fewer cold
    launches), its roofline fraction and the dense fp16 reference."""
    w = build_workload(name, torch, ada, W)
    kept, pages_by_tier, max_row, n_pages, units = workload_shape(w, ada)
    cfg = ada.make_config(w["P"], w["Hq"], w["Hkv"], decode_chunk_pages=args.chunk_pages)
    m = measure_decode(args, w, ada, torch, cfg, kept, max_row, n_pages, units, args.steps, min(args.cold_steps, 20))
    achieved = m["alg_bytes"] / (m["kernel_ms"] * 1e-3) / 1e9
    rec = {
        "config": {"batch": w["B"], "q_heads": w["Hq"], "kv_heads": w["Hkv"], "head_dim": 128,
                   "context_max": int(w["ctx_len"].max()), "context_total": int(w["ctx_len"].sum()),
                   "page_size": w["P"], "kept_token_heads": m["kept"],
                   "kept_by_tier": [kept[t] for t in TIERS], "pages_by_tier": m["pages_by_tier"]},
        "value": m["kept"] / (m["ms_per_step"] * 1e-3), "unit": "KV token-heads/s",
        "value_p10": m["value_p10"], "value_p90": m["value_p90"],
        "ms_per_step": m["ms_per_step"],
        "kernel_ms": m["kernel_ms"], "kernel_ms_event_median": m["kernel_ms_event_median"],
        "algorithmic_bytes": m["alg_bytes"], "achieved_gbps": achieved, "frac": achieved / PEAK_HBM_GBPS,
        "frac_of_read_probe": achieved / read_probe_gbps,
        "frac_of_chunk_probe": achieved / chunk_probe_gbps,
        "traffic": measured_traffic(name),
        "reduce_kernel_ms": m["reduce_kernel_ms"],
        "cold_kernel_ms_median": m["cold_kernel_ms_median"],
        "context_tokens_per_s": m["context_tokens_per_s"],
        # bytes the decode reads per context token-head (dropped tokens cost nothing)
        "bytes_per_context_token_head": m["alg_bytes"] / (float(w["ctx_len"].sum()) * w["Hkv"]),
    }
    if not args.no_dense:
        d = dense_reference(w, ada, torch, cfg)
        d["bytes_per_context_token_head"] = DENSE_TOKEN_BYTES
        rec["dense_fp16_reference"] = d
    del w
    release(torch)
    return rec


def measure_decode(args, w, ada, torch, cfg, kept, max_row, n_pages, units, steps, cold_steps):
    """Pack the workload, then time K decode steps back to back (the value),
    the same K steps with events around each (spread), the split-K kernel
    alone (roofline), the reduction alone, a graph replay of the step and
    cold launches."""
    P, Hq, Hkv, B = w["P"], w["Hq"], w["Hkv"], w["B"]
    tiers = w["tiers"]
    kept_total = sum(kept.values())
    pages_by_tier = {t: 0 for t in TIERS}
    for t in TIERS:
        for b in range(B):
            for h in range(Hkv):
                pages_by_tier[t] += -(-int((tiers[b, h] == t).sum()) // P)
    cache = ada.Cache(cfg, B, max_row, n_pages, units)
    ada.cache_init(cache)
    keys = torch.from_numpy(w["keys"]).cuda()
    vals = torch.from_numpy(w["values"].view(np.int16)).cuda()
    ada.pack(cache, w["ctx_len"], torch.from_numpy(tiers).cuda(), keys, vals)
    st = ada.read_status(cache.status)
    assert st == ada.OK, ada.status_str(st)
    del keys, vals
    release(torch)

    Q = args.queries
    if Q == 1:
        q = torch.from_numpy(w["q"]).cuda()
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        ws = ada.decode_workspace(cache, B)
    else:   # multi-query decode: Q seeded N(0,1) queries per sequence
        qm = np.random.default_rng(4242).standard_normal((B, Q, Hq, 128), dtype=np.float32)
        q = torch.from_numpy(qm).cuda()
        out = torch.empty((B, Q, Hq, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Q, Hq), dtype=torch.float32, device="cuda")
        ws = ada.decode_multi_workspace(cache, B, Q)

    def split_k():
        if Q == 1:
            ada.decode_partials(cache, q, w["scale"], ws)
        else:   # the multi-query call includes its reduction pass
            ada.decode_multi(cache, q, w["scale"], out, lse, ws)

    def step(ev=None):
        if ev is None and Q == 1:   # one library call: the split-K pass and its reduction
            ada.decode(cache, q, w["scale"], out, lse, ws)
            return
        if ev is not None:
            ev[0].record()
        split_k()
        if ev is not None:
            ev[1].record()
        if Q == 1:
            ada.decode_reduce(cache, B, out, lse, ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K back-to-back steps, as a serving loop issues
    # them (no timing events between the launches: an event on the stream
    # adds about 10 us per step of GPU-side gaps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    # spread of the headline: the same back-to-back steps in batches of ten,
    # events only at the batch boundaries (per-step events would add their
    # own gaps), one mean per batch
    batch = 10
    nb = max(2, steps // batch)
    bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nb)]
    for k in range(nb):
        bev[k][0].record()
        for _ in range(batch):
            step()
        bev[k][1].record()
    torch.cuda.synchronize()
    batch_ms = np.array([e0_.elapsed_time(e1_) / batch for e0_, e1_ in bev])
    # the same K steps again with events bracketing every split-K launch and
    # every whole step
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step_events = (time.perf_counter() - t0) * 1e3 / steps
    k_each = [e[0].elapsed_time(e[1]) for e in evs]
    step_each_ms = [e[0].elapsed_time(e[2]) for e in evs]
    k_ms_each = float(np.mean(k_each))
    # dominant kernel alone: K back-to-back split-K launches between two events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        split_k()
    e1.record()
    torch.cuda.synchronize()
    k_ms = e0.elapsed_time(e1) / steps
    # the reduction pass alone, K back-to-back launches (mostly launch cost:
    # behind a split-K launch it adds about 2 us)
    r_ms = None
    if Q == 1:
        e0.record()
        for _ in range(steps):
            ada.decode_reduce(cache, B, out, lse, ws)
        e1.record()
        torch.cuda.synchronize()
        r_ms = e0.elapsed_time(e1) / steps

    # the same step captured once in a HIP graph and replayed K times (a
    # serving loop's form: no per-launch host work between the kernels)
    graph_ms = None
    if Q == 1:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / steps
        del graph

    # cold steps: before each, 1 GiB of another buffer is streamed through the
    # caches with a read kernel (the 256 MB last-level cache then holds clean
    # lines of that buffer, so no write-back is charged to the decode)
    cold = []
    if cold_steps:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        fsink = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(cold_steps):
            ada.probe_read(flush, 1 << 30, 0, fsink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            split_k()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush

    # radius + codes + values per kept token-head, page metadata and table
    # entry per page, the query read and the output written per query row
    alg_bytes = sum(kept[t] * TIER_TOKEN_BYTES[t] for t in TIERS) + 12 * n_pages + B * Q * Hq * 128 * 4 * 2
    step_each = np.array(step_each_ms)
    del cache, ws
    release(torch)
    return {
        "kept": kept_total, "pages_by_tier": [pages_by_tier[t] for t in TIERS], "alg_bytes": alg_bytes,
        "ms_per_step": ms_step, "kernel_ms": k_ms, "kernel_ms_event_mean": k_ms_each,
        "kernel_ms_event_median": float(np.median(k_each)), "reduce_kernel_ms": r_ms,
        "value_p10": kept_total / (float(np.percentile(batch_ms, 90)) * 1e-3),
        "value_p90": kept_total / (float(np.percentile(batch_ms, 10)) * 1e-3),
        "ms_per_step_event_p10": float(np.percentile(step_each, 10)),
        "ms_per_step_event_p90": float(np.percentile(step_each, 90)),
        "graph_ms_per_step": graph_ms, "ms_per_step_with_events": ms_step_events,
        "step_hbm_gbps": alg_bytes / (ms_step * 1e-3) / 1e9,
        "context_tokens_per_s": float(w["ctx_len"].sum()) * Hkv / (ms_step * 1e-3),
        "cold_kernel_ms_median": float(np.median(cold)) if cold else None,
        "cold_gbps": alg_bytes / (np.median(cold) * 1e-3) / 1e9 if cold else None,
    }


def utility_bench(args, w, ada, torch, cfg, kept, max_row, n_pages, units):
    """ada_decode_utility (decode + every kept token's attention mass) against
    ada_decode on the same packed cache."""
    P, Hq, Hkv, B = w["P"], w["Hq"], w["Hkv"], w["B"]
    cache = ada.Cache(cfg, B, max_row, n_pages, units)
    ada.cache_init(cache)
    ada.pack(cache, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), torch.from_numpy(w["keys"]).cuda(),
             torch.from_numpy(w["values"].view(np.int16)).cuda())
    assert ada.read_status(cache.status) == ada.OK
    release(torch)
    q = torch.from_numpy(w["q"]).cuda()
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    util = torch.zeros((n_pages, P), dtype=torch.float32, device="cuda")
    wsu = ada.decode_utility_workspace(cache, B)
    wsd = ada.decode_workspace(cache, B)
    runs = {"utility": lambda: ada.decode_utility(cache, q, w["scale"], util, out, lse, wsu),
            "decode": lambda: ada.decode(cache, q, w["scale"], out, lse, wsd)}
    timing = {}
    for name, fn in runs.items():
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        timing[name] = e0.elapsed_time(e1) / args.steps
    kept_total = sum(kept.values())
    print(json.dumps({
        "metric": "ADA decode with per-token utility emission",
        "value": kept_total / (timing["utility"] * 1e-3), "unit": "KV token-heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": timing["utility"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "page_size": P,
                   "kept_token_heads": kept_total},
        "utility_ms_per_step": timing["utility"], "decode_ms_per_step": timing["decode"],
        "overhead": timing["utility"] / timing["decode"] - 1.0,
    }), flush=True)


def repack_bench(args, w, ada, torch, cfg, kept, max_row, n_pages, units):
    """ada_repack of the packed cache into a second cache under budgets of
    args.repack times each sequence's current bytes, with the utilities of one
    ada_decode_utility step.  Each timed step resets the destination
    (ada_cache_init) and re-packs; the destination is checked against the
    budget afterwards.  With --repack-mask the destination tiers are the
    mask's (56: fp16 tiers re-packed into V8 tiers)."""
    P, Hq, Hkv, B = w["P"], w["Hq"], w["Hkv"], w["B"]
    if args.repack_mask:
        cfg = ada.make_config(P, Hq, Hkv, rdr_tier_mask=args.repack_mask, value_tiers=True)
    src = ada.Cache(cfg, B, max_row, n_pages, units)
    dst = ada.Cache(cfg, B, max_row, n_pages, units)
    ada.cache_init(src)
    ada.pack(src, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), torch.from_numpy(w["keys"]).cuda(),
             torch.from_numpy(w["values"].view(np.int16)).cuda())
    assert ada.read_status(src.status) == ada.OK
    release(torch)
    util = torch.zeros((n_pages, P), dtype=torch.float32, device="cuda")
    ada.decode_utility(src, torch.from_numpy(w["q"]).cuda(), w["scale"], util)
    rate = TIER_TOKEN_BYTES
    cur = [sum(rate[t] * int((w["tiers"][b] == t).sum()) for t in TIERS) for b in range(B)]
    budget = [int(args.repack * c) for c in cur]
    ws = ada.repack_workspace(src, B)

    def step():
        ada.cache_init(dst)
        ada.repack(src, B, util, budget, dst, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert ada.read_status(dst.status) == ada.OK
    h = dst.host()
    kept_total = sum(kept.values())
    kept_after = {t: 0 for t in TIERS}
    used = [0] * B
    for row in range(B * Hkv):
        for page in h["page_table"][row, : h["num_pages"][row]]:
            t, c = int(h["page_meta"][page, 0]), int(h["page_meta"][page, 1])
            kept_after[t] += c
            used[row // Hkv] += rate[t] * c
    assert all(u <= bd for u, bd in zip(used, budget))
    print(json.dumps({
        "metric": "ADA RDR re-pack of a packed cache",
        "value": kept_total / (ms * 1e-3), "unit": "source KV token-heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "page_size": P,
                   "budget_fraction": args.repack, "kept_token_heads_before": kept_total,
                   "rdr_tier_mask": cfg.rdr_tier_mask or 7,
                   "kept_by_tier_before": {str(t): kept[t] for t in TIERS},
                   "kept_by_tier_after": {str(t): kept_after[t] for t in TIERS}},
        "bytes_before": sum(cur), "bytes_after": sum(used), "budget_bytes": sum(budget),
    }), flush=True)


def setup_bench(args, w, ada, torch, W, cfg, kept, max_row, n_pages, units):
    """The setup path: ada_pack of the workload's tier map into an empty cache
    (every kept key encoded exactly, pages placed), each timed step resetting
    the cache first; and ada_rdr_assign on the rdr128k utilities and budgets
    (the ordered RDR selection over every (head, position) of 4 x 128k)."""
    P, Hkv, B = w["P"], w["Hkv"], w["B"]
    cache = ada.Cache(cfg, B, max_row, n_pages, units)
    keys = torch.from_numpy(w["keys"]).cuda()
    vals = torch.from_numpy(w["values"].view(np.int16)).cuda()
    tiers = torch.from_numpy(w["tiers"]).cuda()

    def pack_step():
        ada.cache_init(cache)
        ada.pack(cache, w["ctx_len"], tiers, keys, vals)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    pack_ms = timed(pack_step)
    assert ada.read_status(cache.status) == ada.OK
    kept_total = sum(kept.values())
    del cache, keys, vals, tiers
    release(torch)

    r = W.config("rdr128k")
    rcfg = ada.make_config(r["P"], r["Hq"], r["Hkv"])
    util = torch.from_numpy(r["utility"]).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_out = torch.empty(util.shape, dtype=torch.int8, device="cuda")
    rdr_ms = timed(lambda: ada.rdr_assign(rcfg, r["ctx_len"], util, r["budget"], status, t_out))
    assert ada.read_status(status) == ada.OK
    items = int(r["ctx_len"].sum()) * r["Hkv"]
    print(json.dumps({
        "metric": "ADA setup path: pack (exact encoding + page placement) and RDR assignment",
        "value": kept_total / (pack_ms * 1e-3), "unit": "packed KV token-heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": pack_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "page_size": P,
                   "kept_token_heads": kept_total},
        "rdr_assign": {"workload": "rdr128k", "ms": rdr_ms, "items": items,
                       "items_per_s": items / (rdr_ms * 1e-3)},
    }), flush=True)


def append_bench(args, w, ada, torch, cfg, kept, max_row, n_pages, units):
    """One decode step with one new token per (sequence, KV head): the fused
    ada_decode_append against ada_encode_append followed by ada_decode, each
    on its own copy of the packed cache with room for the appended tokens.
    The new tokens go to the 4-bit tier; keys, values and queries are seeded
    N(0,1) draws."""
    P, Hq, Hkv, B = w["P"], w["Hq"], w["Hkv"], w["B"]
    rows = B * Hkv
    n_steps = args.warmup + args.steps
    extra = rows * (-(-n_steps // P) + 1)               # new pages the appends may open
    caches = []
    keys = torch.from_numpy(w["keys"]).cuda()
    vals = torch.from_numpy(w["values"].view(np.int16)).cuda()
    for _ in range(2):
        c = ada.Cache(cfg, B, max_row + extra // rows, n_pages + extra, units + extra * ada.block_bytes(0, P) // 16)
        ada.cache_init(c)
        ada.pack(c, w["ctx_len"], torch.from_numpy(w["tiers"]).cuda(), keys, vals)
        assert ada.read_status(c.status) == ada.OK
        caches.append(c)
    del keys, vals
    release(torch)
    rng = np.random.default_rng(77)
    nk = torch.from_numpy(rng.standard_normal((n_steps, B, Hkv, 128), dtype=np.float32)).cuda()
    nv = torch.from_numpy(rng.standard_normal((n_steps, B, Hkv, 128)).astype(np.float16).view(np.int16)).cuda()
    nt = torch.ones((B, Hkv), dtype=torch.uint8, device="cuda")
    qs = torch.from_numpy(rng.standard_normal((n_steps, B, Hq, 128), dtype=np.float32)).cuda()
    seq = torch.arange(B, dtype=torch.int32, device="cuda").repeat_interleave(Hkv)
    head = torch.arange(Hkv, dtype=torch.int32, device="cuda").repeat(B)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    wsf = ada.decode_append_workspace(caches[0], B)
    wsd = ada.decode_workspace(caches[1], B)
    sz = ada.append_workspace_bytes(caches[1], rows)
    wsa = torch.empty(max(1, sz), dtype=torch.uint8, device="cuda")

    def fused(i):
        ada.decode_append(caches[0], qs[i], w["scale"], nk[i], nv[i], nt, out, lse, wsf)

    def separate(i):
        ada.encode_append(caches[1], seq, head, nt.reshape(-1), nk[i].reshape(-1, 128), nv[i].reshape(-1, 128), wsa)
        ada.decode(caches[1], qs[i], w["scale"], out, lse, wsd)

    timing = {}
    for name, fn in (("fused", fused), ("separate", separate)):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.warmup, n_steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        timing[name] = e0.elapsed_time(e1) / args.steps
    for c in caches:
        assert ada.read_status(c.status) == ada.OK
    kept_total = sum(kept.values())
    print(json.dumps({
        "metric": "ADA decode step with append (one new token per sequence and KV head)",
        "value": (kept_total + rows) / (timing["fused"] * 1e-3), "unit": "KV token-heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": timing["fused"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "page_size": P,
                   "kept_token_heads_before": kept_total, "new_tier": "T4"},
        "fused_ms_per_step": timing["fused"],
        "append_then_decode_ms_per_step": timing["separate"],
        "speedup": timing["separate"] / timing["fused"],
    }), flush=True)


def dense_reference(w, ada, torch, cfg):
    """Same-box dense fp16 paged decode over the un-dropped keys and values
    (every context token kept, keys rounded to fp16)."""
    from workloads import dense_pages
    B, Hq = w["B"], w["Hq"]
    k16 = w["keys"].astype(np.float16).view(np.uint16)
    kp, vp, pt = dense_pages(k16, w["values"], w["P"])
    del k16
    kp_d = torch.from_numpy(kp.view(np.int16)).cuda()
    vp_d = torch.from_numpy(vp.view(np.int16)).cuda()
    del kp, vp
    pt_d = torch.from_numpy(pt).cuda()
    ctx_d = torch.from_numpy(w["ctx_len"]).cuda()
    q = torch.from_numpy(w["q"]).cuda()
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = ada.dense_workspace(cfg, B, pt.shape[1])
    for _ in range(5):
        ada.dense_decode(cfg, pt_d, ctx_d, kp_d, vp_d, q, w["scale"], out, lse, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record()
    for _ in range(n):
        ada.dense_decode(cfg, pt_d, ctx_d, kp_d, vp_d, q, w["scale"], out, lse, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    token_heads = int(w["ctx_len"].sum()) * w["Hkv"]
    dbytes = token_heads * DENSE_TOKEN_BYTES + B * Hq * 1024
    del kp_d, vp_d
    release(torch)
    gbps = dbytes / (ms * 1e-3) / 1e9
    # frac: the dense step's bytes over its time against the 8 TB/s peak,
    # beside the ADA kernel's roofline fraction
    return {"ms_per_step": ms, "token_heads": token_heads, "bytes_per_token_head": DENSE_TOKEN_BYTES,
            "algorithmic_bytes": dbytes, "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS,
            "token_heads_per_s": token_heads / (ms * 1e-3)}


def cpu_baseline(w, kept_total, max_row, n_pages, units, min_seconds=10.0, max_steps=20):
    """The fp64 CPU oracle, as it stands, decoding the same workload on the
    host's cores (pages built by the oracle's own pack, untimed).  Decode
    steps over the whole batch are repeated until about min_seconds of CPU
    work have been timed."""
    from oracle import oracle as O
    # the host share of one GPU is at most 16 cores, whatever the affinity mask shows
    cores = min(16, len(os.sched_getaffinity(0)))
    B = w["B"]
    oc = O.Cache(w["P"], w["Hq"], w["Hkv"], B, max_row, n_pages, units)
    assert O.pack(oc, w["ctx_len"], w["tiers"], w["keys"], w["values"], nthreads=cores) == O.OK
    steps, dt = 0, 0.0
    while steps < max_steps and (steps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        O.decode(oc, w["q"], w["scale"], nthreads=cores)
        dt += time.perf_counter() - t0
        steps += 1
    # one thread, one decode step of sequence 0 only
    one = O.Cache(w["P"], w["Hq"], w["Hkv"], 1, max_row, n_pages, units)
    assert O.pack(one, w["ctx_len"][:1], w["tiers"][:1], w["keys"][:1], w["values"][:1], nthreads=cores) == O.OK
    kept0 = int((w["tiers"][0, :, : int(w["ctx_len"][0])] >= 0).sum())
    t0 = time.perf_counter()
    O.decode(one, w["q"][:1], w["scale"], nthreads=1)
    dt1 = time.perf_counter() - t0
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": kept_total * steps / dt, "unit": "KV token-heads/s", "cores": cores, "kind": "oracle",
            "seconds": dt, "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "sample": f"{steps} decode steps over all {B} sequences (all heads, all kept tokens, "
                      f"{kept_total} token-heads per step), same queries each step",
            "single_thread": {"value": kept0 / dt1, "seconds": dt1,
                              "sample": f"one decode step of sequence 0 ({kept0} token-heads) on 1 thread"}}


if __name__ == "__main__":
    main()
