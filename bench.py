"""Throughput of one score -> select -> compact pass of attention-score KV-cache
eviction on one MI355X, on seeded synthetic inputs.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--path fused|separate]
                    [--no-cpu-baseline]

(--workload h2o_stream_870 times the H2O decode step instead: one
kvev_h2o_step launch per decoded token of every sequence.  --workload
vtok_reclaim_64k times vToken's liveness marks and lazy reclamation of one
64000-token layer; --workload snap_ring_870 times SnapKV's decode-time ring
buffer step; --workload h2o_decode_4k times H2O's decode-time accumulation:
256 steps of accumulated scoring over a growing 4096-token cache, then one
selection and compaction to the budget.  --hbm-probe measures the plain HBM
read rate of the GPU with the probe library instead.)

A step is the whole eviction path for one layer's cache: scoring (SnapKV
window sum + max-pool over the last W prompt queries), selection (budget,
protected recent window) and compaction (in-place repack, emptied blocks to
the free list).  The default path is the fused call kvev_evict; --path
separate times kvev_score, kvev_select and kvev_compact called one after the
other (same results).  Every step works on its own pristine copy of the cache,
prepared before the timed region, so the timed region holds only the
eviction kernels; L2 and the Infinity Cache are flushed before it starts,
so the keys come from HBM (the flush only reads, so no dirty lines are
left for the timed kernels to write back).

Prints one JSON line: value = scored KV tokens per second (batch x context
tokens, every KV head scored, selected and compacted), plus the HBM roofline
of the dominant kernel (the scoring kernel, timed alone through kvev_score
with HIP events on its launch stream) and the CPU oracle timed on the host
cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="snapkv_prefill_32k")
    ap.add_argument("--path", choices=("fused", "separate"), default="fused")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", action="store_true",
                    help="only run the timed steps (for rocprofv3 runs)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="measure the plain HBM read rate instead (libkvev_probe.so over a "
                         "1 GiB buffer: contiguous, 4 KiB blocks in order, 4 KiB blocks "
                         "through a shuffled list), one JSON line (not the benchmark's metric)")
    ap.add_argument("--overlap-probe", action="store_true",
                    help="measure how much fp32 VALU work overlaps the MFMA units (libkvev_probe.so, "
                         "one workgroup per CU, two waves per SIMD), one JSON line (not the "
                         "benchmark's metric)")
    ap.add_argument("--window-attn", action="store_true",
                    help="time the window forward helper (kvev_window_attn: LSE, and the "
                         "output for DropKV) on the workload's cache and window instead, one "
                         "JSON line (not the benchmark's metric)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


API_SRC = os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc", "api.hip")


def source_hash(path):
    """sha256 (16 hex digits) of a kernel source followed by api.hip, which
    sets the kernel's launch shape (tiles, workgroup size)."""
    h = hashlib.sha256(open(path, "rb").read())
    h.update(open(API_SRC, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload, kernel_src, kernel="score", sha_key="score_source_sha256_16"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source and launch code."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get(sha_key) != source_hash(kernel_src):
        return None
    return d.get("hbm_bytes_per_launch")


def read_pass_traffic(workload):
    """HBM bytes per fused pass (score kernel + evict_finish_kernel) from the
    committed counter summary, if taken on the current kernel and launch code."""
    p = os.path.join(ROOT, "profiles", f"pass_{workload}_hbm_counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    h = hashlib.sha256()
    for f in ("score.hip", "finish.hip", "api.hip"):
        h.update(open(os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc", f), "rb").read())
    if d.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    return d.get("hbm_bytes_per_pass")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import kv_cache_eviction_qk_amd as K
    import synth

    K.load_library()  # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.hbm_probe:
        return bench_hbm_probe(args)
    if args.overlap_probe:
        return bench_overlap_probe(args)
    cfg = synth.CONFIGS[args.workload]
    if args.window_attn:
        return bench_window_attn(args, cfg)
    if args.workload == "h2o_stream_870":
        return bench_h2o_stream(args, cfg)
    if args.workload == "vtok_reclaim_64k":
        return bench_vtok(args, cfg)
    if args.workload == "snap_ring_870":
        return bench_ring_stream(args, cfg)
    if args.workload == "h2o_decode_4k":
        return bench_decode_accumulate(args, cfg)
    if cfg.decode_steps:
        print(json.dumps({"error": f"{args.workload} is a decode schedule, not a one-shot pass"}))
        sys.exit(2)
    kind = cfg.flags[0]
    flag = {"sum": K.SUM, "pool": K.POOL, "drop": K.DROP}[kind]
    steps, warm = args.steps, args.warmup
    copies = max(steps, warm)

    t0 = time.time()
    case = synth.make_case(cfg)
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    pristine = K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                       dev(case["seq_len"]), dev(case["pos"]))
    q, q_pos = dev(case["q"]), dev(case["q_pos"])
    B, Hkv, G, W, D = cfg.B, cfg.Hkv, cfg.G, cfg.W, cfg.D
    # forward-pass outputs for the window: LSE (and a for DropKV), made by the helper kernel
    ws_wa = K.new_workspace(pristine, G, W)
    lse, a = K.window_attn(pristine, q, q_pos, cfg.softmax_scale, G, ws_wa, want_a=(kind == "drop"))
    torch.cuda.synchronize()
    del ws_wa
    log("window LSE ready")

    # one pristine copy of the mutable cache state per step
    caches = []
    for i in range(copies):
        caches.append(K.Cache(pristine.k_pool.clone(), pristine.v_pool.clone(),
                              pristine.block_table.clone(), pristine.seq_len.clone(),
                              pristine.pos.clone()))
    nb = case["num_blocks"]
    free_lists = [torch.full((nb,), -1, dtype=torch.int32, device="cuda") for _ in range(copies)]
    free_counts = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(copies)]
    ws = K.new_workspace(pristine, G, W)  # room for split windows
    score_out = pristine.score_buffer()
    victims = torch.empty((B, Hkv, pristine.max_slots), dtype=torch.int32, device="cuda")
    n_victims = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    stats = torch.zeros(5, dtype=torch.int64, device="cuda")
    scrub = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")  # 1 GiB

    def restore(i):
        c = caches[i]
        c.k_pool.copy_(pristine.k_pool)
        c.v_pool.copy_(pristine.v_pool)
        c.block_table.copy_(pristine.block_table)
        c.seq_len.copy_(pristine.seq_len)
        c.pos.copy_(pristine.pos)
        free_lists[i].fill_(-1)
        free_counts[i].zero_()

    def flush_caches():
        # Read 1 GiB: evicts L2 and the 256 MB Infinity Cache without leaving
        # dirty lines behind (a write-back flood would slow the timed kernels).
        return scrub.sum()

    outs = {"sum": None, "pooled": None, "drop": None}
    outs[{"sum": "sum", "pool": "pooled", "drop": "drop"}[kind]] = score_out

    def step_fused(i):
        K.evict(caches[i], q, lse, q_pos, cfg.softmax_scale, G, flag, cfg.budget, cfg.recent,
                score_out, victims, n_victims, free_lists[i], free_counts[i], ws,
                pool_kernel=cfg.pool_kernel, a=a, stats=stats)

    def step(i, ev=None):
        if ev is None and args.path == "fused":
            step_fused(i)
            return
        c = caches[i]
        if ev is not None:
            ev[0].record()
        K.score(c, q, lse, q_pos, cfg.softmax_scale, G, flag, cfg.pool_kernel, sum=outs["sum"],
                pooled=outs["pooled"], drop=outs["drop"], a=a, workspace=ws)
        if ev is not None:
            ev[1].record()
        K.select(c, score_out, cfg.budget, cfg.recent, victims, n_victims, ws)
        if ev is not None:
            ev[2].record()
        K.compact(c, victims, n_victims, free_lists[i], free_counts[i], ws, stats)
        if ev is not None:
            ev[3].record()

    def warm_path(fused):
        for i in range(warm):
            if fused:
                step_fused(i)
            else:
                step(i, [torch.cuda.Event() for _ in range(4)])
        torch.cuda.synchronize()

    # warm both paths (first launches load code objects); the timed path last
    warm_path(args.path != "fused")
    for i in range(warm):
        restore(i)
    warm_path(args.path == "fused")
    st = stats.cpu().numpy().tolist()
    for i in range(copies):
        restore(i)
    flush_caches()
    torch.cuda.synchronize()
    log(f"warmup done; stats of one pass {st}")

    # ---- timed region: exactly `steps` passes
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = e0.elapsed_time(e1)
    if args.profile_steps:
        log(f"profile run done: {ms_total / steps:.4f} ms/step")
        return
    ms_step = ms_total / steps
    tokens = B * cfg.L
    value = tokens * steps / (ms_total / 1e3)

    st = stats.cpu().numpy().tolist()
    nv = n_victims.cpu().numpy()
    # block-level waste of the pass's eviction, by kvev_measure on the last
    # step's victims: naive (holes left in place) vs after compaction
    waste = K.measure(pristine.seq_len, victims, n_victims)

    # ---- each pass timed on its own, after a restore and a cache flush of its
    # own (the keys come from HBM every time): median, p10 and p90
    per_pass_us = None
    if args.path == "fused":
        for i in range(steps):
            restore(i)
        ts = []
        for i in range(steps):
            flush_caches()
            q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            q0.record()
            step(i)
            q1.record()
            torch.cuda.synchronize()
            ts.append(q0.elapsed_time(q1) * 1e3)
        ts = np.array(ts)
        per_pass_us = {"median": float(np.median(ts)), "p10": float(np.percentile(ts, 10)),
                       "p90": float(np.percentile(ts, 90)), "n": int(steps)}

    # ---- the scoring kernel alone (kvev_score, same launch configuration):
    # `steps` back-to-back launches between two HIP events on their stream,
    # each reading its own copy of the cache after one flush, so its keys
    # come from HBM
    for i in range(steps):
        restore(i)
    flush_caches()
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(steps):
        K.score(caches[i], q, lse, q_pos, cfg.softmax_scale, G, flag, cfg.pool_kernel,
                sum=outs["sum"], pooled=outs["pooled"], drop=outs["drop"], a=a, workspace=ws)
    s1.record()
    torch.cuda.synchronize()
    t_score_alone = s0.elapsed_time(s1) / steps

    # ---- the separate calls with an event between stages (same work again)
    flush_caches()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    t_score = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    t_select = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    t_compact = sum(e[2].elapsed_time(e[3]) for e in evs) / steps

    # ---- the fused passes of independent caches (the layers of one model)
    # alternating between two streams, each with its own workspace and outputs:
    # one layer's latency-bound selection and compaction overlap the next
    # layer's scoring.  Reported beside the headline, which is one stream.
    two_stream_ms, two_stream_same = None, None
    if args.path == "fused" and steps >= 2:
        for i in range(steps):
            restore(i)
        side = [dict(ws=ws, score=score_out, vic=victims, nv=n_victims, st=stats),
                dict(ws=K.new_workspace(pristine, G, W), score=pristine.score_buffer(),
                     vic=torch.empty_like(victims), nv=torch.empty_like(n_victims),
                     st=torch.zeros_like(stats))]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        cur = torch.cuda.current_stream()

        def two_stream_passes(k):
            for sx in streams:
                sx.wait_stream(cur)
            for i in range(k):
                sd = side[i % 2]
                with torch.cuda.stream(streams[i % 2]):
                    K.evict(caches[i], q, lse, q_pos, cfg.softmax_scale, G, flag, cfg.budget,
                            cfg.recent, sd["score"], sd["vic"], sd["nv"], free_lists[i],
                            free_counts[i], sd["ws"], pool_kernel=cfg.pool_kernel, a=a,
                            stats=sd["st"])
            for sx in streams:
                cur.wait_stream(sx)

        # the first launches on new streams are slow: warm them up first
        two_stream_passes(min(steps, max(warm, 2)))
        torch.cuda.synchronize()
        for i in range(steps):
            restore(i)
        flush_caches()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(cur)
        two_stream_passes(steps)
        t1.record(cur)
        torch.cuda.synchronize()
        two_stream_ms = t0.elapsed_time(t1) / steps
        two_stream_same = side[1]["st"].cpu().numpy().tolist() == st
        del side, streams

    # algorithmic bytes (what the method must move; see the design notes)
    ms_ = pristine.max_slots
    eb = 2 if cfg.dtype == "bf16" else 4
    units = B * Hkv
    n = cfg.L
    key_bytes = units * n * D * eb
    val_bytes = key_bytes if kind == "drop" else 0
    rows = G * W
    q_bytes = B * Hkv * rows * D * eb * (2 if kind == "drop" else 1) + B * Hkv * rows * 4
    pos_bytes = units * n * 4
    bt_bytes = units * math.ceil(n / 16) * 4
    out_bytes = units * n * 4
    score_bytes = key_bytes + val_bytes + q_bytes + pos_bytes + bt_bytes + out_bytes
    n_vic = int(nv.sum())
    cand = units * max(0, n - cfg.recent)
    select_bytes = cand * 4 + n_vic * 4
    rows_moved = int(st[1])
    compact_bytes = n_vic * 4 + rows_moved * 2 * D * eb * 2 + rows_moved * 4 * 2
    pass_bytes = score_bytes + select_bytes + compact_bytes
    achieved = score_bytes / (t_score_alone / 1e3) / 1e9
    src = os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc", "score.hip")
    traffic = read_traffic(args.workload, src)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, cfg, kind)

    out = {
        "metric": ("scored KV tokens/sec (score+select+compact) at 32K ctx; % of peak HBM GB/s"
                   if args.workload == "snapkv_prefill_32k" else
                   f"scored KV tokens/sec (score+select+compact) at {cfg.L} tokens; "
                   "% of peak HBM GB/s"),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": {"spans": "synthetic (seeded; spans planted on window-query directions)",
                 "heavy_hitters": "synthetic (seeded; 2% heavy hitters planted on the query "
                                  "direction)",
                 "near_mean": "synthetic (seeded; 10% near-mean value rows)",
                 "iid": "synthetic (seeded; iid normal rows)"}[cfg.recipe],
        "config": {"workload": args.workload, "path": args.path, "batch": B, "kv_heads": Hkv,
                   "group": G,
                   "head_dim": D, "context": n, "obs_window": W, "pool_kernel": cfg.pool_kernel,
                   "budget": cfg.budget, "recent_window": cfg.recent, "score": kind,
                   "block_size": 16, "accumulate": "fp32"},
        "pipeline_hbm_frac": pass_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "pipeline_bytes": pass_bytes,
        # the whole timed pass (the metric's scope) against HBM: the pass's
        # algorithmic bytes over ms_per_step; "roofline" below is the
        # dominant kernel's alone
        "pass_roofline": {"scope": f"one {args.path} pass (score + select + compact)",
                          "bound": "hbm", "achieved": pass_bytes / (ms_step / 1e3) / 1e9,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": pass_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
                          "algorithmic_bytes": pass_bytes, "ms": ms_step,
                          "traffic": (read_pass_traffic(args.workload)
                                      if args.path == "fused" else None)},
        # every KV head of every scored token: B * Hkv * L head-rows a pass
        "head_rows_per_s": B * Hkv * n * steps / (ms_total / 1e3),
        # each pass alone, after its own flush (not the headline, which is the
        # back-to-back passes)
        "per_pass_us": per_pass_us,
        "separate_calls_ms": {"score": t_score, "select": t_select, "compact": t_compact},
        # fused passes of independent caches alternating on two streams (not the headline)
        "two_stream_ms_per_pass": two_stream_ms,
        "two_stream_stats_equal": two_stream_same,
        "wall_s": wall,
        "blocks_freed_per_pass": int(st[0]),
        "block_waste": {k: waste[k] for k in ("F_naive", "F_after", "frac_le_half_naive",
                                              "frac_le_half_after")},
        "rows_moved_per_pass": rows_moved,
        "roofline": {"kernel": "score_kernel (kvev_score)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": score_bytes, "launch_ms": t_score_alone},
        # the compaction call (prep + gather) of the separate-call passes: where
        # many kept rows move, it outlasts the scoring
        "compact_roofline": {"call": "kvev_compact (prep + gather + in-order)", "bound": "hbm",
                             "achieved": compact_bytes / (t_compact / 1e3) / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": compact_bytes / (t_compact / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": read_traffic(
                                 args.workload,
                                 os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc",
                                              "compact.hip"),
                                 kernel="compact", sha_key="source_sha256_16"),
                             "algorithmic_bytes": compact_bytes, "call_ms": t_compact},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_h2o_stream(args, cfg):
    """The H2O decode lifecycle, one kvev_h2o_step launch per step over every
    KV head (the new token's attention output, score accumulation, pruning to the
    budget, overwrite in place).  The stream's first budget - L steps fill the
    cache (untimed, with the warmup steps); the timed steps each prune one
    token per head.  value = decoded tokens (one per sequence) per second."""
    import numpy as np
    import torch

    import kv_cache_eviction_qk_amd as K
    import synth

    B, Hkv, G, D = cfg.B, cfg.Hkv, cfg.G, cfg.D
    fill = cfg.budget - cfg.L
    warm = args.warmup
    steps = min(args.steps, cfg.decode_steps - fill - warm)
    if steps < 1:
        print(json.dumps({"error": f"{cfg.decode_steps} steps in the stream: lower --warmup"}))
        sys.exit(2)
    case = synth.make_case(cfg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    cache = K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                    dev(case["seq_len"]), dev(case["pos"]))
    score = cache.score_buffer()
    free_list = torch.full((case["num_blocks"],), -1, dtype=torch.int32, device="cuda")
    free_count = torch.zeros(1, dtype=torch.int32, device="cuda")
    total = fill + warm + steps
    qs, ks, vs = [], [], []
    for i in range(total):  # every step's inputs resident before the timed region
        q, _ = synth.make_queries(cfg, 0, 1, case["dirs"], step=i)
        k, v = synth.decode_token_kv(case, i)
        qs.append(dev(q.reshape(B, cfg.Hq, D)))
        ks.append(dev(k))
        vs.append(dev(v))
    tpos = [torch.full((B,), cfg.L + i, dtype=torch.int32, device="cuda") for i in range(total)]
    evicted = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    attn = torch.empty((B, cfg.Hq, D), dtype=torch.float32, device="cuda")
    ws = K.new_h2o_workspace(cache, G, cfg.budget)

    def step(i, with_attn=True):
        K.h2o_step(cache, qs[i], ks[i], vs[i], tpos[i], G, cfg.softmax_scale, score, cfg.budget,
                   cfg.recent, free_list, free_count, ws, evicted,
                   attn_out=attn if with_attn else None)

    for i in range(fill + warm):
        step(i)
    torch.cuda.synchronize()
    assert int(cache.seq_len.min()) == cfg.budget
    log(f"stream filled to {cfg.budget} tokens per head; {warm} warmup steps")
    # the timed steps as one HIP graph (a decode loop is replayed, not
    # re-issued from the host; each step is one kernel); a copy of the state
    # lets the same steps also run eagerly for comparison
    snap = [t.clone() for t in (cache.k_pool, cache.v_pool, cache.block_table, cache.seq_len,
                                cache.pos, score, free_list, free_count)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(fill + warm, total):
            step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / steps
    if args.profile_steps:
        log(f"profile run done: {ms_step:.4f} ms/step")
        return
    ev = evicted.cpu().numpy()
    assert (ev >= 0).all(), "a timed step did not prune"
    after = [t.clone() for t in (cache.k_pool, cache.pos, score)]
    for t, v in zip((cache.k_pool, cache.v_pool, cache.block_table, cache.seq_len, cache.pos,
                     score, free_list, free_count), snap):
        t.copy_(v)
    torch.cuda.synchronize()
    x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x0.record()
    for i in range(fill + warm, total):
        step(i)
    x1.record()
    torch.cuda.synchronize()
    ms_eager = x0.elapsed_time(x1) / steps
    same = all(bool(torch.equal(a, b)) for a, b in zip(after, (cache.k_pool, cache.pos, score)))
    assert same, "graph replay and eager steps differ"
    # the same steps without the attention output (value rows not read)
    for t, v in zip((cache.k_pool, cache.v_pool, cache.block_table, cache.seq_len, cache.pos,
                     score, free_list, free_count), snap):
        t.copy_(v)
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2):
        for i in range(fill + warm, total):
            step(i, with_attn=False)
    torch.cuda.synchronize()
    for t, v in zip((cache.k_pool, cache.v_pool, cache.block_table, cache.seq_len, cache.pos,
                     score, free_list, free_count), snap):
        t.copy_(v)
    torch.cuda.synchronize()
    y0, y1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    y0.record()
    graph2.replay()
    y1.record()
    torch.cuda.synchronize()
    ms_no_attn = y0.elapsed_time(y1) / steps
    # algorithmic bytes of one step (the launch is the whole step)
    eb = 2 if cfg.dtype == "bf16" else 4
    units, n = B * Hkv, cfg.budget
    step_bytes = (2 * units * n * D * eb            # cached keys and values
                  + B * cfg.Hq * D * 4              # attention output
                  + B * cfg.Hq * D * eb             # query rows
                  + units * n * (4 + 4 + 4)         # scores read and written, positions read
                  + units * math.ceil(n / 16) * 4   # block ids
                  + units * 2 * D * eb * 2)         # new K / V row, read and written
    achieved = step_bytes / (ms_step / 1e3) / 1e9
    traffic = read_traffic(args.workload,
                           os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc", "h2o_step.hip"),
                           kernel="h2o_step", sha_key="source_sha256_16")
    cpu = None if args.no_cpu_baseline else cpu_baseline_h2o(case, cfg, fill)
    out = {
        "metric": "H2O decode steps: tokens/sec (attention output + score accumulation + prune + "
                  "in-place overwrite per step)",
        "value": B / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; 2% heavy hitters planted on the query direction)",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "group": G,
                   "head_dim": D, "budget": cfg.budget, "recent_window": cfg.recent,
                   "start_tokens": cfg.L, "block_size": 16, "accumulate": "fp32"},
        "wall_s": wall,
        "timing": "one HIP graph of the timed steps, replayed once",
        "eager_ms_per_step": ms_eager,
        "ms_per_step_without_attention_output": ms_no_attn,
        "roofline": {"kernel": "h2o_step_kernel (kvev_h2o_step)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": step_bytes, "launch_ms": ms_step},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_decode_accumulate(args, cfg):
    """H2O decode-time accumulation on the 4096-token decode shape (B8, 8 KV
    heads x 4, D128, bf16): one schedule is 256 decode steps, each one
    kvev_score launch (SUM | ACCUMULATE, one query row per head) over the
    grown cache, then kvev_select and kvev_compact to the budget (870 tokens,
    435 recent).  The step's LSE is the attention forward's output in a
    model; here kvev_window_attn computes every step's LSE before the timed
    region.  The cache holds every decoded token's row from the start; a
    step's token joins by its length.  value = scored KV tokens (batch x
    cached tokens, summed over the steps) per second."""
    import numpy as np
    import torch

    import kv_cache_eviction_qk_amd as K
    import synth

    B, Hkv, G, D = cfg.B, cfg.Hkv, cfg.G, cfg.D
    T = cfg.decode_steps
    case = synth.make_case(cfg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    cache = K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                    dev(case["seq_len"]), dev(case["pos"]))
    ws = K.new_workspace(cache, G, 1)
    # one cache view per step (its own length tensor), so the steps need no
    # copies between launches and the schedule can be captured as a graph
    qs, qps, lses, views = [], [], [], []
    for t in range(T):  # every step's query and LSE resident before the timed region
        q, qp = synth.make_queries(cfg, 0, 1, case["dirs"], step=t)
        qs.append(dev(q))
        qps.append(dev(qp))
        n_t = torch.full((B, Hkv), cfg.L + t + 1, dtype=torch.int32, device="cuda")
        views.append(K.Cache(cache.k_pool, cache.v_pool, cache.block_table, n_t, cache.pos))
        lse, _ = K.window_attn(views[-1], qs[-1], qps[-1], cfg.softmax_scale, G, ws)
        lses.append(lse.clone())
    final_len = torch.full((B, Hkv), cfg.L_final, dtype=torch.int32, device="cuda")
    final = K.Cache(cache.k_pool, cache.v_pool, cache.block_table, final_len, cache.pos)
    torch.cuda.synchronize()
    score = cache.score_buffer()
    state = (cache.k_pool, cache.v_pool, cache.block_table, cache.pos, final_len)
    snap = [t.clone() for t in state]
    free_list = torch.full((case["num_blocks"] + 8,), -1, dtype=torch.int32, device="cuda")
    free_count = torch.zeros(1, dtype=torch.int32, device="cuda")
    vic = torch.empty((B, Hkv, cache.max_slots), dtype=torch.int32, device="cuda")
    nv = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    stats = torch.zeros(5, dtype=torch.int64, device="cuda")

    def scoring():
        score.zero_()
        for t in range(T):
            K.score(views[t], qs[t], lses[t], qps[t], cfg.softmax_scale, G, K.SUM | K.ACCUMULATE,
                    1, sum=score, workspace=ws)

    def schedule():
        scoring()
        K.select(final, score, cfg.budget, cfg.recent, vic, nv, ws)
        K.compact(final, vic, nv, free_list, free_count, ws, stats=stats, score_row=score)

    def restore():
        for t, v in zip(state, snap):
            t.copy_(v)
        free_count.zero_()

    schedule()          # warm, and the selection's persistent state exercised once
    restore()
    torch.cuda.synchronize()
    g_sched, g_score = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_sched):
        schedule()
    with torch.cuda.graph(g_score):
        scoring()
    torch.cuda.synchronize()
    reps = max(1, min(args.steps, 5))
    total_ms = wall = score_ms = 0.0
    for _ in range(reps):
        restore()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record()
        g_sched.replay()
        e1.record()
        torch.cuda.synchronize()
        wall += time.perf_counter() - w0
        total_ms += e0.elapsed_time(e1)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        g_score.replay()
        s1.record()
        torch.cuda.synchronize()
        score_ms += s0.elapsed_time(s1)
    ms_sched = total_ms / reps
    ms_score = score_ms / reps / T   # a score launch (plus the zero fill spread over the steps)
    # the graph-replayed schedule matches an eager one
    restore()
    schedule()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (score, vic, nv, cache.k_pool, cache.pos)]
    restore()
    g_sched.replay()
    torch.cuda.synchronize()
    assert all(bool(torch.equal(a, b)) for a, b in zip(eager, (score, vic, nv, cache.k_pool,
                                                              cache.pos))), "graph != eager"
    st = stats.cpu().numpy()
    assert int(st[4]) == 0 and int(nv.min()) == cfg.L_final - cfg.budget, (st, nv.min())
    if args.profile_steps:
        log(f"profile run done: {ms_sched:.3f} ms/schedule, score {ms_score * 1e3:.2f} us")
        return
    eb = 2 if cfg.dtype == "bf16" else 4
    units = B * Hkv
    scored = B * sum(cfg.L + t + 1 for t in range(T))
    # one score launch at the mean length: K rows, positions, block ids, the
    # score read and written (ACCUMULATE), the query rows and LSE
    n_mean = sum(cfg.L + t + 1 for t in range(T)) / T
    launch_bytes = (units * n_mean * (D * eb + 4 + 8) + units * math.ceil(n_mean / 16) * 4
                    + B * cfg.Hq * D * eb + B * cfg.Hq * 4)
    achieved = launch_bytes / (ms_score / 1e3) / 1e9
    out = {
        "metric": "H2O decode-time accumulation: scored KV tokens/sec (256 accumulated scoring "
                  "steps + select + compact per schedule)",
        "value": scored / (ms_sched / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": max(1, args.warmup),
        "ms_per_step": ms_sched,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; 2% heavy hitters planted on the query direction)",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "group": G,
                   "head_dim": D, "context": f"{cfg.L} -> {cfg.L_final}", "decode_steps": T,
                   "budget": cfg.budget, "recent_window": cfg.recent, "score": "sum+accumulate",
                   "block_size": 16},
        "wall_s": wall,
        "timing": "a step is one whole schedule (256 score launches, then select and compact) "
                  "captured as one HIP graph and replayed between HIP events; the 256 score "
                  "launches alone as a second graph for the per-launch time",
        "score_launch_us": ms_score * 1e3,
        "blocks_freed": int(st[0]),
        "roofline": {"kernel": "score_kernel (kvev_score, SUM | ACCUMULATE, one query row)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": read_traffic(args.workload, os.path.join(
                         ROOT, "kv_cache_eviction_qk_amd", "csrc", "score.hip"),
                         kernel="score", sha_key="source_sha256_16"),
                     "algorithmic_bytes": launch_bytes, "launch_ms": ms_score},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_decode(case, cfg),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(case, cfg):
    """The oracle's accumulated scoring on the host cores for a bounded
    sample: the first 8 decode steps of the schedule (its own LSE per step,
    excluded from the timing), every head."""
    import numpy as np

    import oracle
    import synth
    B, Hkv = cfg.B, cfg.Hkv
    threads = baseline_threads(B * Hkv)
    acc = np.zeros((B, Hkv, case["max_blocks"] * 16), np.float32)
    steps, scored, dt = 8, 0, 0.0
    for t in range(steps):
        n = cfg.L + t + 1
        q, q_pos = synth.make_queries(cfg, 0, 1, case["dirs"], step=t)
        st = dict(case, seq_len=np.full((B, Hkv), n, np.int32), q=q, q_pos=q_pos, W=1)
        lse64, _ = oracle.lse_a(st, nthreads=threads)
        t0 = time.perf_counter()
        o = oracle.score(st, lse64.astype(np.float32), oracle.SUM | oracle.ACCUMULATE, 1,
                         prev_sum=acc, nthreads=threads)["sum"]
        dt += time.perf_counter() - t0
        acc = np.nan_to_num(o, nan=0.0).astype(np.float32)
        scored += B * n
    return {"value": scored / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {steps} accumulated scoring steps of all {B * Hkv} KV heads; "
                      f"{dt:.1f} s (select and compact not included)", **host_cpu()}


def bench_ring_stream(args, cfg):
    """SnapKV's decode-time ring buffer, one kvev_ring_step launch per step
    over every KV head (softmax weights into the rings, pooled ring sums,
    one token dropped per head at the budget).  The first budget - L steps
    fill the cache (untimed, with the warmup steps); every timed step drops
    one token per head.  Every seventh step of a sequence is a null step.
    value = decoded tokens (one per sequence) per second."""
    import numpy as np
    import torch

    import kv_cache_eviction_qk_amd as K
    import synth

    B, Hkv, G, D, W = cfg.B, cfg.Hkv, cfg.G, cfg.D, cfg.W
    fill = cfg.budget - cfg.L
    warm = args.warmup
    steps = min(args.steps, cfg.decode_steps - fill - warm)
    if steps < 1:
        print(json.dumps({"error": f"{cfg.decode_steps} steps in the stream: lower --warmup"}))
        sys.exit(2)
    case = synth.make_case(cfg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    cache = K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                    dev(case["seq_len"]), dev(case["pos"]))
    rs = K.RingState(cache, W)
    free_list = torch.full((case["num_blocks"],), -1, dtype=torch.int32, device="cuda")
    free_count = torch.zeros(1, dtype=torch.int32, device="cuda")
    total = fill + warm + steps
    qs, ks, vs, obs = [], [], [], []
    for i in range(total):  # every step's inputs resident before the timed region
        q, _ = synth.make_queries(cfg, 0, 1, case["dirs"], step=i)
        k, v = synth.decode_token_kv(case, i)
        qs.append(dev(q.reshape(B, cfg.Hq, D)))
        ks.append(dev(k))
        vs.append(dev(v))
        obs.append(dev(np.array([int((i + b) % 7 != 3) for b in range(B)], np.int32)))
    tpos = [torch.full((B,), cfg.L + i, dtype=torch.int32, device="cuda") for i in range(total)]
    evicted = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")

    def step(i):
        K.ring_step(cache, rs, qs[i], ks[i], vs[i], tpos[i], obs[i], G, cfg.softmax_scale,
                    cfg.budget, cfg.recent, cfg.pool_kernel, free_list, free_count, evicted)

    for i in range(fill + warm):
        step(i)
    torch.cuda.synchronize()
    assert int(cache.seq_len.min()) == cfg.budget
    log(f"stream filled to {cfg.budget} tokens per head; {warm} warmup steps")
    state = (cache.k_pool, cache.v_pool, cache.block_table, cache.seq_len, cache.pos, rs.hist,
             rs.ring, rs.rank)
    snap = [t.clone() for t in state]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(fill + warm, total):
            step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / steps
    if args.profile_steps:
        log(f"profile run done: {ms_step:.4f} ms/step")
        return
    ev = evicted.cpu().numpy()
    assert (ev >= 0).all(), "a timed step did not drop a token"
    after = [t.clone() for t in state]
    for t, v in zip(state, snap):
        t.copy_(v)
    torch.cuda.synchronize()
    x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x0.record()
    for i in range(fill + warm, total):
        step(i)
    x1.record()
    torch.cuda.synchronize()
    ms_eager = x0.elapsed_time(x1) / steps
    assert all(bool(torch.equal(a, b)) for a, b in zip(after, state)), \
        "graph replay and eager steps differ"
    # algorithmic bytes of one step: per cached token its key row, position,
    # rank (read and written) and ring (obsWindow entries read, one written);
    # per head the query rows and the new token's key and value rows
    eb = 2 if cfg.dtype == "bf16" else 4
    units, n = B * Hkv, cfg.budget
    step_bytes = (units * n * (D * eb + 4 + 8 + 4 * W + 4)
                  + units * math.ceil(n / 16) * 4
                  + B * cfg.Hq * D * eb
                  + units * 3 * D * eb)
    achieved = step_bytes / (ms_step / 1e3) / 1e9
    traffic = read_traffic(args.workload,
                           os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc", "ring_step.hip"),
                           kernel="ring_step", sha_key="source_sha256_16")
    cpu = None if args.no_cpu_baseline else cpu_baseline_ring(case, cfg, fill)
    out = {
        "metric": "SnapKV ring-buffer decode steps: tokens/sec (ring weights + pooled ring sums "
                  "+ drop + in-place overwrite per step)",
        "value": B / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; 2% heavy hitters planted on the query direction)",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "group": G,
                   "head_dim": D, "budget": cfg.budget, "recent_window": cfg.recent,
                   "obs_window": W, "pool_kernel": cfg.pool_kernel, "start_tokens": cfg.L,
                   "null_steps": "every seventh step of a sequence", "block_size": 16},
        "wall_s": wall,
        "timing": "one HIP graph of the timed steps, replayed once",
        "eager_ms_per_step": ms_eager,
        "roofline": {"kernel": "ring_step_kernel (kvev_ring_step)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": step_bytes, "launch_ms": ms_step},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_ring(case, cfg, fill):
    """The oracle's ring step on the host (one thread), for a bounded sample:
    the fill steps untimed, then 12 dropping steps timed."""
    import numpy as np

    import oracle
    import synth
    st = oracle.ring_state(dict(case), cfg.W)

    def one(i):
        q, _ = synth.make_queries(cfg, 0, 1, case["dirs"], step=i)
        k, v = synth.decode_token_kv(case, i)
        obs = np.array([int((i + b) % 7 != 3) for b in range(cfg.B)], np.int32)
        return oracle.ring_step(st, q.reshape(cfg.B, cfg.Hq, cfg.D), k, v,
                                np.full(cfg.B, cfg.L + i, np.int32), obs, cfg.budget, cfg.recent,
                                cfg.pool_kernel)[0]
    for i in range(fill):
        st = one(i)
    n = 12
    t0 = time.perf_counter()
    for i in range(fill, fill + n):
        st = one(i)
    dt = time.perf_counter() - t0
    return {"value": cfg.B * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} dropping steps of all {cfg.B * cfg.Hkv} KV heads at {cfg.budget} "
                      f"tokens; {dt:.1f} s", **host_cpu()}


def _vtok_bytes(U, rows, nsrc, alloc_blocks, row_bytes):
    """Algorithmic HBM bytes of one reclamation call.  Per moved row: K and V
    read and written (4 x row_bytes), its position read, staged, read back and
    written (16).  Per source block: its 16 liveness bytes read and written,
    source and offset records written and read (16), block id read, rewritten
    and pushed (12), live count written (4).  Per allocated block of a head:
    block id and live count read by the plan (8)."""
    return rows * (4 * row_bytes + 16) + nsrc * (32 + 16 + 12 + 4) + alloc_blocks * 8



def bench_hbm_probe(args):
    """Plain read rate of this GPU's HBM: every byte of a 1 GiB buffer read
    once per launch, for three access shapes and a sweep of loads in flight
    and grid sizes.  Each launch is timed with HIP events on the stream it
    runs on, after a 1 GiB read of another buffer has evicted L2 and the
    Infinity Cache; the median of `reps` launches is reported."""
    import numpy as np
    import torch

    from kv_cache_eviction_qk_amd import build as kbuild

    path = kbuild.PROBE_OUT
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run python -m kv_cache_eviction_qk_amd.build")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.kvev_probe_read.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_size_t, P,
                                  ctypes.c_int, P, P]
    L.kvev_probe_read.restype = ctypes.c_int
    nbytes = 1 << 30
    nblk = nbytes // 4096
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")  # xor of the words: 0
    scrub = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    perm = np.random.default_rng(0).permutation(nblk).astype(np.int32)
    assert perm.min() == 0 and perm.max() == nblk - 1
    lists = {"identity": torch.arange(nblk, dtype=torch.int32, device="cuda"),
             "shuffled": torch.from_numpy(perm).cuda()}
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    reps = max(3, args.steps if args.steps <= 9 else 5)
    shapes = (("contiguous", 0, None), ("4KiB blocks in order", 1, "identity"),
              ("4KiB blocks shuffled", 1, "shuffled"))
    rows, best = [], {}
    for name, pattern, lst in shapes:
        lp = lists[lst].data_ptr() if lst else None
        for depth in (4, 8, 16):
            for grid in (1024, 2048, 4096, 8192):
                ts = []
                for _ in range(reps):
                    scrub.sum()
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    rc = L.kvev_probe_read(pattern, depth, buf.data_ptr(), nbytes, lp, grid,
                                           sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
                    e1.record(stream)
                    torch.cuda.synchronize()
                    if rc != 0:
                        raise RuntimeError(f"kvev_probe_read returned {rc}")
                    ts.append(e0.elapsed_time(e1) / 1e3)
                t = sorted(ts)[len(ts) // 2]
                gbs = nbytes / t / 1e9
                rows.append({"shape": name, "depth": depth, "grid": grid, "us": t * 1e6,
                             "GB/s": round(gbs, 1)})
                log(f"{name:22s} depth {depth:2d} grid {grid:5d}: {gbs:7.1f} GB/s")
                if gbs > best.get(name, (0,))[0]:
                    best[name] = (round(gbs, 1), depth, grid)
    assert int(sink.item()) == 0
    print(json.dumps({"metric": "hbm_read_rate", "unit": "GB/s", "bytes_per_launch": nbytes,
                      "reps": reps, "peak": HBM_PEAK_GBS,
                      "best": {k: {"GB/s": v[0], "depth": v[1], "grid": v[2],
                                   "frac_of_peak": round(v[0] / HBM_PEAK_GBS, 3)}
                               for k, v in best.items()},
                      "sweep": rows}), flush=True)

def bench_overlap_probe(args):
    """How much fp32 VALU work overlaps the MFMA units: the probe library's
    overlap kernel (256 workgroups of 8 waves, one per CU) in six modes, each
    timed with HIP events on its launch stream (best of 3), reported as ns
    per iteration of the probe's loop; then the barrier probe (does a
    workgroup barrier wait for outstanding stores?), in ns per round."""
    import torch

    from kv_cache_eviction_qk_amd import build as kbuild

    path = kbuild.PROBE_OUT
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run python -m kv_cache_eviction_qk_amd.build")
    L = ctypes.CDLL(path)
    L.kvev_probe_overlap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.kvev_probe_overlap.restype = ctypes.c_int
    grid, iters = 256, 20000
    out = torch.zeros(grid * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    names = ["8 MFMA a wave", "32 FMA a wave", "8 MFMA + 32 FMA, same wave",
             "8 MFMA on even waves, 32 FMA on odd waves", "16 exp2 + 16 mul a wave",
             "8 MFMA + 16 exp2 + 16 mul, same wave"]
    res = {}
    for mode in range(6):
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = L.kvev_probe_overlap(mode, grid, iters, out.data_ptr(),
                                      ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"kvev_probe_overlap returned {rc}")
            ts.append(e0.elapsed_time(e1) * 1e-3)
        res[names[mode]] = round(min(ts) * 1e9 / iters, 2)
        log(f"{names[mode]:45s} {res[names[mode]]:8.2f} ns/iteration")
    # and whether a workgroup barrier waits for the waves' outstanding stores
    L.kvev_probe_barrier.argtypes = L.kvev_probe_overlap.argtypes
    L.kvev_probe_barrier.restype = ctypes.c_int
    bgrid, biters = 256, 2000
    bout = torch.zeros(bgrid * 1024, dtype=torch.float32, device="cuda")
    bnames = ["LDS exchange between barriers", "a nontemporal store before each barrier",
              "the store and an explicit s_waitcnt vmcnt(0)"]
    bres = {}
    for mode in range(3):
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = L.kvev_probe_barrier(mode, bgrid, biters, bout.data_ptr(),
                                      ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"kvev_probe_barrier returned {rc}")
            ts.append(e0.elapsed_time(e1) * 1e-3)
        bres[bnames[mode]] = round(min(ts) * 1e9 / biters, 1)
        log(f"{bnames[mode]:45s} {bres[bnames[mode]]:8.1f} ns/round")
    print(json.dumps({"metric": "mfma_valu_overlap", "unit": "ns per iteration", "grid": grid,
                      "threads": 512, "iterations": iters, "modes": res,
                      "barrier_ns_per_round": bres, "barrier_grid": bgrid,
                      "barrier_threads": 1024}), flush=True)

def bench_window_attn(args, cfg):
    """kvev_window_attn on the workload's prompt cache (every head at length L)
    and window (G x W rows per KV head; W = 1 for the decode workloads, one
    decode step's query): the LSE, plus the output for DropKV.  Algorithmic
    bytes: the keys (and values when the output is wanted) read once, the
    queries read, the LSE and output written; partials excluded."""
    import numpy as np
    import torch

    import kv_cache_eviction_qk_amd as K
    import synth
    case = synth.make_case(cfg)
    want_a = cfg.flags[0] == "drop"

    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    dc = K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                 dev(case["seq_len"]), dev(case["pos"]))
    q, qp = dev(case["q"]), dev(case["q_pos"])
    G, W, D = cfg.G, cfg.W, cfg.D
    ws = K.new_workspace(dc, G, W)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    a = torch.empty(q.shape, dtype=torch.float32, device="cuda") if want_a else None
    for _ in range(args.warmup):
        K.window_attn(dc, q, qp, cfg.softmax_scale, G, ws, want_a=want_a, lse_out=lse, a_out=a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        K.window_attn(dc, q, qp, cfg.softmax_scale, G, ws, want_a=want_a, lse_out=lse, a_out=a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    units = cfg.B * cfg.Hkv
    eb = 2 if cfg.dtype == "bf16" else 4
    tokens = int(case["seq_len"].sum())
    rows = units * G * W
    nbytes = tokens * D * eb * (2 if want_a else 1) + rows * D * eb + rows * 4 * (1 + (D if want_a else 0))
    print(json.dumps({"kernel": "window_attn", "workload": cfg.name, "rows_per_kv_head": G * W,
                      "tokens": tokens, "want_a": want_a, "ms_per_call": ms,
                      "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / ms / 1e6,
                      "hbm_frac": nbytes / ms / 1e6 / HBM_PEAK_GBS, "steps": args.steps}),
          flush=True)


def bench_vtok(args, cfg):
    """vToken on one 64000-token layer (B16, 8 KV heads, D128, bf16): a step
    restores the layer's token table (block lists, positions, liveness, the
    free list: device copies, about 50 MB), marks half of every head's tokens
    dead (kvev_vtok_evict, the victims of a uniform random policy) and runs
    one lazy reclamation whose source batch covers the head (kvev_vtok_reclaim,
    theta_F = 0.25).  value = KV tokens covered per second (batch x heads x
    context / step time)."""
    import numpy as np
    import torch

    import kv_cache_eviction_qk_amd as K
    import synth

    B, Hkv, D = cfg.B, cfg.Hkv, cfg.D
    U = B * Hkv
    theta, max_sources = 0.25, 4096
    steps, warm = args.steps, args.warmup
    t0 = time.time()
    spare = U * ((cfg.budget + 15) // 16 + 1)      # room for every head's destinations
    case = synth.make_case(cfg, spare_blocks=spare)
    vic, nv = synth.random_victims(case, cfg.budget, cfg.recent)
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    cache = K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                    dev(case["seq_len"]), dev(case["pos"]))
    ms = cache.max_slots
    nblk = case["max_blocks"]
    live0 = torch.zeros((B, Hkv, ms), dtype=torch.uint8, device="cuda")
    live0[:, :, :cfg.L] = 1
    bl0 = torch.zeros((B, Hkv, nblk), dtype=torch.int32, device="cuda")
    bl0[:, :, :cfg.L // 16] = 16
    used = np.zeros(case["num_blocks"], bool)
    used[case["block_table"][case["block_table"] >= 0]] = True
    free_ids = np.flatnonzero(~used).astype(np.int32)
    fl0 = torch.full((case["num_blocks"],), -1, dtype=torch.int32, device="cuda")
    fl0[:free_ids.size] = dev(free_ids)
    fc0 = torch.tensor([free_ids.size], dtype=torch.int32, device="cuda")
    bt0, pos0 = cache.block_table.clone(), cache.pos.clone()
    live, bl = live0.clone(), bl0.clone()
    fl, fc = fl0.clone(), fc0.clone()
    vic_d, nv_d = dev(vic), dev(nv)
    ws = K.new_vtok_workspace(cache, max_sources)
    ews = K.new_vtok_evict_workspace(cache)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    stats = torch.zeros(10, dtype=torch.int64, device="cuda")
    evs = []

    def step(timed):
        for t, v in ((cache.block_table, bt0), (cache.pos, pos0), (live, live0), (bl, bl0),
                     (fl, fl0), (fc, fc0)):
            t.copy_(v)
        K.vtok_evict(cache, live, bl, vic_d, nv_d, ews, status)
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
        K.vtok_reclaim(cache, live, bl, theta, max_sources, fl, fc, ws, stats=stats)
        if timed:
            b.record()
            evs.append((a, b))

    for _ in range(warm):
        step(False)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    assert int(status.item()) == 0 and st[0] == U and st[1] == 0, st
    w0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step(True)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / steps
    ms_reclaim = sum(a.elapsed_time(b) for a, b in evs) / steps
    if args.profile_steps:
        log(f"profile run done: {ms_step:.4f} ms/step, reclaim {ms_reclaim:.4f} ms")
        return
    # the online checks of I1 and I2 around one more step, timed on their own
    cws = K.new_vtok_check_workspace(cache)
    for t, v in ((cache.block_table, bt0), (cache.pos, pos0), (live, live0), (bl, bl0),
                 (fl, fl0), (fc, fc0)):
        t.copy_(v)
    K.vtok_evict(cache, live, bl, vic_d, nv_d, ews, status)
    c0, c1, c2, c3 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    c0.record()
    dig0 = K.vtok_digest(cache, live)
    c1.record()
    K.vtok_reclaim(cache, live, bl, theta, max_sources, fl, fc, ws, stats=stats)
    dig1 = K.vtok_digest(cache, live).clone()
    c2.record()
    chk = K.vtok_check(cache, live, bl, fl, fc, cws)
    c3.record()
    mws = torch.empty(K.load_library().kvev_vtok_map_workspace_bytes(
        ctypes.byref(cache.struct())), dtype=torch.uint8, device="cuda")
    K.vtok_slot_mapping(cache, live, mws)  # warm
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record()
    _, _, mcount = K.vtok_slot_mapping(cache, live, mws)
    m1.record()
    torch.cuda.synchronize()
    online = {"I1_digests_equal": bool(torch.equal(dig0, dig1)),
              "I2_check": chk.cpu().tolist(), "digest_ms": c0.elapsed_time(c1),
              "check_ms": c2.elapsed_time(c3), "slot_mapping_ms": m0.elapsed_time(m1),
              "mapped_tokens": int(mcount.sum().item())}
    assert online["mapped_tokens"] == U * cfg.budget, online
    assert online["I1_digests_equal"] and online["I2_check"] == [0, 0, 0, 0], online
    st = stats.cpu().numpy()
    # the plan's sizes from the marks, on the host (accounting only), checked
    # against the call's own statistics
    nb_head = (cfg.L + 15) // 16
    nsrc = rows = dests = 0
    for u in range(U):
        b, h = divmod(u, Hkv)
        dead = np.bincount(vic[b, h, :nv[b, h]] // 16, minlength=nblk)[:nb_head]
        cnt = 16 - dead
        cand = np.flatnonzero(cnt[:nb_head - 1] < 16)[:max_sources]
        t = int(cnt[cand].sum())
        nsrc += cand.size
        rows += t
        dests += (t + 15) // 16
    assert rows == int(st[4]) and nsrc - dests == int(st[3]), (rows, nsrc, dests, st)
    row_bytes = D * (2 if cfg.dtype == "bf16" else 4)
    call_bytes = _vtok_bytes(U, rows, nsrc, U * nb_head, row_bytes)
    achieved = call_bytes / (ms_reclaim / 1e3) / 1e9
    traffic = read_traffic(args.workload,
                           os.path.join(ROOT, "kv_cache_eviction_qk_amd", "csrc", "vtoken.hip"),
                           kernel="vtok_reclaim", sha_key="source_sha256_16")
    cpu = None if args.no_cpu_baseline else cpu_baseline_vtok(cfg, theta, max_sources)
    out = {
        "metric": "vToken marks + lazy reclamation: KV tokens/sec covered (one 64000-token "
                  "layer, half the tokens dead)",
        "value": U * cfg.L / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic (seeded; uniform random victims, 16 recent protected)",
        "config": {"workload": args.workload, "batch": B, "kv_heads": Hkv, "head_dim": D,
                   "context": cfg.L, "victims_per_head": cfg.L - cfg.budget,
                   "recent_window": cfg.recent, "theta_F": theta, "source_batch": max_sources,
                   "block_size": 16},
        "wall_s": wall,
        "timing": "HIP events around the timed steps (table restore + marks + reclamation); "
                  "the reclamation call alone between events of its own",
        "reclaim_ms": ms_reclaim,
        "blocks_freed": int(st[3]),
        "rows_moved": int(st[4]),
        "bytes_moved": int(st[5]),
        "online_checks": online,
        "roofline": {"kernel": "kvev_vtok_reclaim (plan, admit, move, apply launches)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": call_bytes, "launch_ms": ms_reclaim},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_vtok(cfg, theta, max_sources):
    """The oracle's marks and reclamation on the host (one thread), on a
    bounded sample: a two-sequence slice (16 KV heads) of the same shape."""
    import numpy as np

    import oracle
    import synth
    sub = cfg.scaled(B=2)
    U = sub.B * sub.Hkv
    case = synth.make_case(sub, spare_blocks=U * ((sub.budget + 15) // 16 + 1))
    vic, nv = synth.random_victims(case, sub.budget, sub.recent)
    st = dict(case)
    st["live"], st["block_live"] = oracle.vtok_liveness(case)
    used = np.zeros(case["num_blocks"], bool)
    used[case["block_table"][case["block_table"] >= 0]] = True
    free_ids = np.flatnonzero(~used).astype(np.int32)
    fl = np.full(case["num_blocks"], -1, np.int32)
    fl[:free_ids.size] = free_ids
    reps = 0
    t0 = time.perf_counter()
    while True:
        st2, _ = oracle.vtok_evict(st, vic, nv)
        oracle.vtok_reclaim(st2, theta, max_sources, fl, free_ids.size)
        reps += 1
        dt = time.perf_counter() - t0
        if dt > 10.0 or reps >= 8:
            break
    return {"value": U * sub.L * reps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x marks + reclamation of {U} of {cfg.B * cfg.Hkv} KV heads "
                      f"(a 2-sequence slice, {sub.L} tokens each); {dt:.1f} s", **host_cpu()}


def cpu_baseline_h2o(case, cfg, fill):
    """The oracle's decode step on the host (one thread: it walks the heads in
    order), for a bounded sample: the fill steps untimed, then 24 pruning
    steps timed."""
    import numpy as np

    import oracle
    import synth
    st = dict(case)
    st["score"] = np.zeros((cfg.B, cfg.Hkv, case["max_blocks"] * 16), np.float32)
    fl = np.full(case["num_blocks"], -1, np.int32)

    def one(i):
        q, _ = synth.make_queries(cfg, 0, 1, case["dirs"], step=i)
        k, v = synth.decode_token_kv(case, i)
        return oracle.h2o_step(st, q.reshape(cfg.B, cfg.Hq, cfg.D), k, v,
                               np.full(cfg.B, cfg.L + i, np.int32), cfg.budget, cfg.recent,
                               free_list=fl, free_count=0)[0]
    for i in range(fill):
        st = one(i)
    n = 24
    t0 = time.perf_counter()
    for i in range(fill, fill + n):
        st = one(i)
    dt = time.perf_counter() - t0
    return {"value": cfg.B * n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} pruning steps of all {cfg.B * cfg.Hkv} KV heads at {cfg.budget} "
                      f"tokens; {dt:.1f} s", **host_cpu()}


def host_cpu():
    """The host CPU's model name and the CPUs this process may run on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_visible": len(os.sched_getaffinity(0))}


def baseline_threads(units):
    """Oracle threads: one head per thread at most, within the host's share
    of 16 CPUs per GPU (the oracle splits its work over heads)."""
    import oracle
    return max(1, min(oracle.default_threads(), units))


def cpu_baseline(case, cfg, kind):
    """The oracle (score + select + compact) on the host cores, on a bounded
    sample of the same workload; its LSE is its own (not the GPU's)."""
    import numpy as np

    import oracle
    units = cfg.B * cfg.Hkv
    threads = baseline_threads(units)
    # every head of the workload when that stays within about 20 thread-seconds
    sample = list(range(units))
    log(f"cpu baseline: oracle on {len(sample)} of {units} KV heads, {threads} threads")
    lse64, a64 = oracle.lse_a(case, want_a=(kind == "drop"), units=sample, nthreads=threads)
    import synth
    lse32 = lse64.astype(np.float32)
    a32 = a64.astype(np.float32) if a64 is not None else None
    flag = {"sum": oracle.SUM, "pool": oracle.POOL, "drop": oracle.DROP}[kind]
    t0 = time.perf_counter()
    out = oracle.score(case, lse32, flag, cfg.pool_kernel, a32=a32, units=sample,
                       nthreads=threads)
    key = {"sum": "sum", "pool": "pooled", "drop": "drop"}[kind]
    s32 = np.nan_to_num(out[key], nan=0.0).astype(np.float32)
    seq = case["seq_len"].copy().reshape(-1)
    mask = np.zeros(units, bool)
    mask[sample] = True
    seq_s = np.where(mask, seq, 0).astype(np.int32)   # heads outside the sample hold no tokens
    vic, nv = oracle.select(s32, seq_s, cfg.budget, cfg.recent)
    sub = dict(case)
    sub["seq_len"] = seq_s.reshape(case["seq_len"].shape)
    oracle.compact(sub, vic, nv)
    dt = time.perf_counter() - t0
    tokens = cfg.L * len(sample) / cfg.Hkv   # scored tokens the sample covers
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(sample)} of {units} KV heads (full context {cfg.L}); "
                      f"{dt:.1f} s of score+select+compact on {threads} threads "
                      f"(about {dt * threads:.0f} thread-seconds)", **host_cpu()}


if __name__ == "__main__":
    main()
