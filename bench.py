"""Benchmark of the CSA2 FP4-cache step on one MI355X.

Default workload: decode at 1,048,576 tokens of context (524,288 compressed
entries, m = 2), batch 1, 64 heads, top-k 2048, 128-row bf16 window, and the
10-layer schedule Full, Reuse, Reindex, Reuse, ... (5 index scans + 5 top-k
selections + 10 attentions + the Full layer's cache write per step).  Inputs are
seeded synthetic data already resident in HBM when timing starts.

Cold mode is the headline: the step rotates over R copies of the cache, with R
chosen so that the bytes the other R - 1 copies' steps touch (indexer keys plus
gathered rows) exceed twice the 256 MB last-level (MALL) cache: when a copy comes
round again its bytes have been pushed out of the MALL.  Warm mode (one copy,
replayed) is reported beside it, and so are the median and 10th / 90th percentile
of single cold steps timed one by one with HIP events.

Prints ONE JSON line: tokens/s (sequences / step time), the FP4 cache bytes read
per step and their rate, a roofline record for the indexer scan (the kernel that
carries the FP4 bytes: HBM-bound in decode, FP4-MFMA-bound in the prefill chunk,
where it is a dense contraction), timed with HIP events on its own stream over
graph replays of back-to-back launches, the same timing for each library call of
the step (in prefill also the attention's bf16 MFMA rate), and the CPU oracle on
a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import functools
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 MFMA, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
INDEX_DIM = 128
LATENT_DIM = 512
IDX_ENTRY_BYTES = 68  # 64 B of E2M1 codes + 4 E8M0 scales per indexer key
MAIN_ENTRY_BYTES = 288  # 256 B of E2M1 codes + 32 E4M3 scales per main entry
MALL_BYTES = 256 << 20
METRIC = "decode tokens/sec & achieved HBM GB/s (FP4 cache) at 1M ctx, top-K 2048"
# sources whose change invalidates a stored counter measurement of the scan kernel
SCAN_SOURCES = ("sparse_attention_fp4_cache_amd/csrc/index_score.hip", "sparse_attention_fp4_cache_amd/csrc/common.hpp",
                "sparse_attention_fp4_cache_amd/csrc/Makefile")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_1m_10layer")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads of the CPU oracle baseline (0: the OpenMP default of the host)")
    p.add_argument("--graph", type=int, default=1, help="replay the step as one HIP graph (1) or launch eagerly (0)")
    p.add_argument("--replicas", type=int, default=0,
                   help="cache copies rotated in cold mode (0: enough that the other copies' touched bytes "
                        "exceed twice the MALL)")
    p.add_argument("--dist-steps", type=int, default=200,
                   help="single cold steps timed one by one for the median and p10 / p90")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="after timing, run one plain device copy of this size (counter calibration)")
    return p.parse_args()


def scan_source_hash() -> str:
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(wl_name: str):
    """HBM bytes per scan launch from the committed counter summary, or None when
    there is none or the scan kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"index_score_traffic_{wl_name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != scan_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def fp4_bytes_per_step(wl):
    if wl.kind == "schedule":  # one token through every layer, one cache per Full layer
        b = 0
        for li, mode in enumerate(wl.modes):
            if mode == "swa":
                continue
            n = int(wl.cache_workload(wl.source(li)).n_entries[0])
            if mode == "full" or (mode == "reindex" and wl.npool == 0):
                b += n * IDX_ENTRY_BYTES
            elif mode == "reindex":
                b += min(8 * wl.npool, n) * IDX_ENTRY_BYTES
            b += min(wl.K, n) * MAIN_ENTRY_BYTES
        return b
    if wl.kind == "prefill":
        return int(wl.n_visible().astype("int64").sum()) * IDX_ENTRY_BYTES + wl.chunk * wl.K * MAIN_ENTRY_BYTES
    n = [int(x) for x in wl.n_entries]
    if wl.npool > 0:  # Reindex layers read only their pool's members
        b = sum(1 for m in wl.layers if m == "full") * sum(n) * IDX_ENTRY_BYTES
        b += sum(1 for m in wl.layers if m == "reindex") * sum(min(8 * wl.npool, x) for x in n) * IDX_ENTRY_BYTES
    else:
        b = sum(1 for m in wl.layers if m in ("full", "reindex")) * sum(n) * IDX_ENTRY_BYTES
    b += len(wl.layers) * sum(min(wl.K, x) for x in n) * MAIN_ENTRY_BYTES
    return b


def touched_bytes_per_step(wl):
    """Cache bytes one step reads from one cache copy: the indexer keys every index
    layer scans (each layer scans the same keys, so they count once) plus the main
    rows the attentions gather (at most k per index layer and sequence)."""
    if wl.kind == "schedule":
        b = 0
        for w in wl.writers():
            n = int(wl.cache_workload(w).n_entries[0])
            layers = [li for li in range(len(wl.modes)) if wl.source(li) == w]
            idx_layers = sum(1 for li in layers if wl.modes[li] in ("full", "reindex"))
            b += n * IDX_ENTRY_BYTES + idx_layers * min(wl.K, n) * MAIN_ENTRY_BYTES
        return b
    if wl.kind == "prefill":
        n = int(wl.n_entries[0]) + wl.n_chunk_entries
        return n * (IDX_ENTRY_BYTES + MAIN_ENTRY_BYTES)
    n = [int(x) for x in wl.n_entries]
    idx_layers = sum(1 for m in wl.layers if m in ("full", "reindex"))
    return sum(n) * IDX_ENTRY_BYTES + idx_layers * sum(min(wl.K, x) for x in n) * MAIN_ENTRY_BYTES


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(wl):
    """The oracle, as it is, on a bounded sample of the workload, scaled to one step.
    Decode: one index layer (scan + top-k) over up to 524,288 entries of the first
    sequence and one attention.  Prefill: two queries of the chunk end to end."""
    import numpy as np

    import oracle
    from sparse_attention_fp4_cache_amd.workloads import small_variant

    if wl.kind == "prefill":
        n = int(wl.n_entries[0]) + wl.n_chunk_entries
        lat, key = wl.cache_rows(0, 0, n)
        c = oracle.Cache(wl.num_slots)
        oracle.fp4_cache_write(c, lat, key, wl.slots(0, 0, n))
        d = wl.layer_inputs(0)
        bt = wl.block_table()
        which = np.array([0, wl.chunk - 1], np.int32)
        nv = wl.n_visible()
        t0 = time.perf_counter()
        sc, _, _ = oracle.index_score(c, d["q_idx"][which], d["w"][which], nv[which], bt,
                                      seq_of_query=np.zeros(2, np.int32))
        idx = np.full((wl.chunk, wl.K), -1, np.int32)
        idx[which] = oracle.topk_select(sc, nv[which], wl.K)
        oracle.sparse_attn_prefill_chunk(c, d["q"], idx, bt[0], d["swa"], d["swa_first_valid"], wl.W,
                                         1.0 / 512 ** 0.5, which=which)
        dt = time.perf_counter() - t0
        return {"value": len(which) / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"2 of the chunk's {wl.chunk} queries (scan, top-{wl.K}, attention), {dt:.2f} s"}

    if wl.kind == "schedule":
        return cpu_baseline_schedule(wl)
    n_full = int(wl.n_entries[0])
    frac = max(1, math.ceil(n_full / 524288))
    sub = small_variant(wl, ctx=[int(wl.ctx[0]) // frac], name=wl.name + "_sample")
    n = int(sub.n_entries[0])
    lat, key = sub.cache_rows(0, 0, n)
    c = oracle.Cache(sub.num_slots)
    oracle.fp4_cache_write(c, lat, key, sub.slots(0, 0, n))
    del lat, key
    d = sub.layer_inputs(0)
    bt = sub.block_table()[:1]
    nv = sub.n_visible()[:1]
    t0 = time.perf_counter()
    sc, _, _ = oracle.index_score(c, d["q_idx"][:1], d["w"][:1], nv, bt)
    idx = oracle.topk_select(sc, nv, sub.K)
    t1 = time.perf_counter()
    oracle.sparse_attn_decode(c, d["q"][:1], idx, bt, d["swa"][:1], d["swa_len"][:1], 1.0 / 512 ** 0.5)
    t2 = time.perf_counter()
    # entries scanned per step: every index layer scans the whole cache, or, with a
    # candidate pool, the Reindex layers only their pool's members
    full_layers = sum(1 for m in wl.layers if m == "full" or (m == "reindex" and wl.npool == 0))
    pool_layers = sum(1 for m in wl.layers if m == "reindex" and wl.npool > 0)
    entries = full_layers * sum(int(x) for x in wl.n_entries)
    entries += pool_layers * sum(min(8 * wl.npool, int(x)) for x in wl.n_entries)
    step_s = (t1 - t0) * entries / n + len(wl.layers) * wl.B * (t2 - t1)
    return {"value": wl.B / step_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"one index layer (MXFP4 scan + top-{wl.K}) over {n} entries and one {wl.H}-head attention "
                       f"({t1 - t0:.2f} s + {t2 - t1:.2f} s), scaled to the step: scans and top-k x{entries / n:g} "
                       f"(entries scanned by all index layers), attention x{len(wl.layers)} layers "
                       f"x{wl.B} sequences")}


def cpu_baseline_schedule(wl):
    """The oracle on one index layer (scan + top-k) over the first 524,288 entries of
    the m = 1 decoder cache and one attention, scaled to the whole schedule's scanned
    entries and attentions."""
    import oracle
    from sparse_attention_fp4_cache_amd.workloads import small_variant

    dec = wl.cache_workload(wl.writers()[-1])
    sub = small_variant(dec, ctx=[524288], name=wl.name + "_sample")
    n = int(sub.n_entries[0])
    lat, key = sub.cache_rows(0, 0, n)
    c = oracle.Cache(sub.num_slots)
    oracle.fp4_cache_write(c, lat, key, sub.slots(0, 0, n))
    del lat, key
    d = wl.query_workload().layer_inputs(wl.writers()[-1])
    bt = sub.block_table()[:1]
    nv = sub.n_visible()[:1]
    t0 = time.perf_counter()
    sc, _, _ = oracle.index_score(c, d["q_idx"], d["w"], nv, bt)
    idx = oracle.topk_select(sc, nv, wl.K)
    t1 = time.perf_counter()
    oracle.sparse_attn_decode(c, d["q"], idx, bt, d["swa"], d["swa_len"], 1.0 / 512 ** 0.5)
    t2 = time.perf_counter()
    entries = 0
    for li, mode in enumerate(wl.modes):
        if mode == "full" or (mode == "reindex" and wl.npool == 0):
            entries += int(wl.cache_workload(wl.source(li)).n_entries[0])
        elif mode == "reindex":
            entries += min(8 * wl.npool, int(wl.cache_workload(wl.source(li)).n_entries[0]))
    step_s = (t1 - t0) * entries / n + len(wl.modes) * (t2 - t1)
    return {"value": 1.0 / step_s, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": (f"one index layer (MXFP4 scan + top-{wl.K}) over {n} entries of the m = 1 cache and one "
                       f"{wl.H}-head attention ({t1 - t0:.2f} s + {t2 - t1:.2f} s), scaled to the schedule: scans "
                       f"x{entries / n:g} (entries scanned by all index layers), attention x{len(wl.modes)} layers")}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; sharding the path over several GPUs "
                                   "is described, not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from sparse_attention_fp4_cache_amd import lib
    from sparse_attention_fp4_cache_amd.step import DecodeStep, PrefillStep, ScheduleDecodeStep
    from sparse_attention_fp4_cache_amd.workloads import WORKLOADS

    if not os.path.exists(lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    lib.load()
    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    Step = {"decode": DecodeStep, "prefill": PrefillStep, "schedule": ScheduleDecodeStep}[wl.kind]
    st = Step(wl, dev)
    st.build_cache()
    torch.cuda.synchronize()
    touched = touched_bytes_per_step(wl)
    R = args.replicas if args.replicas > 0 else 1 + math.ceil(2 * MALL_BYTES / touched)
    # copies of the whole cache: at most 32 and 64 GB of HBM
    R = max(1, min(R, 32, (64 << 30) // max(1, st.cache_bytes())))
    steps = [st] + [st.replica() for _ in range(R - 1)]
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()  # every kernel of the step runs on this stream
    with torch.cuda.stream(stream):
        for s in steps:
            s.run()  # one eager step per copy (the Full layer rewrites its newest entry)
    stream.synchronize()
    graphs = None
    if args.graph:
        graphs = []
        for s in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                s.run()
            graphs.append(g)
        torch.cuda.synchronize()

    def one_step(i, r):
        if graphs is not None:
            graphs[r].replay()
        else:
            steps[r].run()

    def timed(n, rotate):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(n):
                one_step(i, i % R if rotate else 0)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            one_step(i, i % R)
    torch.cuda.synchronize()
    # ---- timed region: K whole steps, cold (rotating cache copies), then warm
    ms_per_step = timed(args.steps, rotate=True)
    warm_ms = timed(args.steps, rotate=False)

    # ---- single cold steps, each between two HIP events on the step's stream
    def step_dist(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            evs[0].record(stream)
            for i in range(n):
                one_step(i, i % R)
                evs[i + 1].record(stream)
        torch.cuda.synchronize()
        t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
        pick = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
        return {"n": n, "median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9), "min_ms": t[0],
                "max_ms": t[-1]}

    dist = step_dist(max(1, args.dist_steps)) if args.dist_steps > 0 else None

    # ---- each library call alone: back-to-back launches over the same inputs as the
    # step (every layer, every cache copy), captured in a graph and timed with HIP
    # events on the stream; the scan (index_score) is the roofline kernel
    def burst_ms(calls, target=60):
        reps = max(2, math.ceil(target / len(calls)))

        def run_all():
            for fn in calls:
                fn()

        with torch.cuda.stream(stream):
            run_all()
        stream.synchronize()
        g = None
        if args.graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                run_all()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                if g is not None:
                    g.replay()
                else:
                    run_all()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(calls)), reps * len(calls)

    calls_us = {}
    if wl.kind == "schedule":
        # the m = 1 decoder cache's Full-layer scan is the roofline kernel (the largest scan)
        wdec = wl.writers()[-1]
        for w in wl.writers():
            Lw = st.layers[w]
            key = "index_topk_m1" if w == wdec else "index_topk_m2"
            if key in calls_us:
                continue
            calls_us[key] = burst_ms([functools.partial(
                lib.index_topk, s.caches[w]["cache"], Lw["q_idx"], Lw["w"], s.caches[w]["n_visible"],
                s.caches[w]["block_table"], s.caches[w]["scores"], wl.K, Lw["topk"], s.caches[w]["ws_topk"])
                for s in steps])[0] * 1e3
        Cd = st.caches[wdec]
        if Cd["pooled"]:
            calls_us["index_pool_build"] = burst_ms([functools.partial(
                lib.index_pool_build, Cd["scores"], Cd["n_visible"], wl.npool, Cd["pool"], Cd["ws_pool"])])[0] * 1e3
            calls_us["index_topk_pool"] = burst_ms([functools.partial(
                lib.index_topk_pool, s.caches[wdec]["cache"], L["q_idx"], L["w"], Cd["n_visible"], Cd["pool"],
                Cd["block_table"], Cd["scores_pool"], wl.K, L["topk"], Cd["ws_topk_pool"])
                for s in steps for L in st.layers if L["mode"] == "reindex"])[0] * 1e3
        calls_us["sparse_attn_decode"] = burst_ms([functools.partial(
            lib.sparse_attn_decode, s.caches[L["src"]]["cache"], L["q"], st.layers[L["src"]]["topk"],
            s.caches[L["src"]]["block_table"], L["swa"], L["swa_len"], st.scale, L["out"], L["lse"], st.ws_attn)
            for s in steps for L in st.layers if L["mode"] != "swa"])[0] * 1e3
        scan = [functools.partial(lib.index_score_counted, s.caches[wdec]["cache"], st.layers[wdec]["q_idx"],
                                  st.layers[wdec]["w"], Cd["n_visible"], Cd["block_table"], Cd["scores"], wl.K,
                                  s.caches[wdec]["ws_topk"])
                for s in steps]
        counted_ws = [s.caches[wdec]["ws_topk"] for s in steps]
        idx_bytes = int(Cd["wl"].n_entries[0]) * IDX_ENTRY_BYTES
        tokens = 1
    elif wl.kind == "decode":
        # layers that scan the whole cache (with a candidate pool, only the Full layer)
        idx_layers = [L for L in st.layers if L["mode"] == "full" or (L["mode"] == "reindex" and wl.npool == 0)]
        if wl.npool > 0:
            calls_us["index_pool_build"] = burst_ms([functools.partial(
                lib.index_pool_build, st.scores, st.n_visible, wl.npool, st.pool, st.ws_pool)])[0] * 1e3
            L0 = st.layers[0]
            calls_us["index_topk_pool_build"] = burst_ms([functools.partial(
                lib.index_topk_pool_build, s.cache, L0["q_idx"], L0["w"], s.n_visible, s.block_table, st.scores,
                wl.K, L0["topk"], wl.npool, st.pool, st.ws_gate) for s in steps])[0] * 1e3
            calls_us["index_topk_pool"] = burst_ms([functools.partial(
                lib.index_topk_pool, s.cache, L["q_idx"], L["w"], s.n_visible, st.pool, s.block_table,
                st.scores_pool, wl.K, L["topk"], st.ws_topk_pool)
                for s in steps for L in st.layers if L["mode"] == "reindex"])[0] * 1e3
        # layer-major over the copies: consecutive calls never read the same copy, so
        # each call finds its keys out of the MALL (cold), as in the step.  The roofline
        # burst runs the scan with the selection's digit counting, the kernel index_topk
        # runs in the step (index_score_counted; the counts pile up in the workspace,
        # which is cleared after the burst).  index_score runs the same kernel with its
        # counts off; it is not timed here, so that every launch of the kernel in this
        # run is a counting one.
        scan = [functools.partial(lib.index_score_counted, s.cache, L["q_idx"], L["w"], s.n_visible, s.block_table,
                                  s.scores, wl.K, s.ws_topk)
                for L in idx_layers for s in steps]
        counted_ws = [s.ws_topk for s in steps]
        calls_us["index_topk"] = burst_ms([functools.partial(lib.index_topk, s.cache, L["q_idx"], L["w"], s.n_visible,
                                                             s.block_table, s.scores, wl.K, L["topk"], s.ws_topk)
                                           for L in idx_layers for s in steps])[0] * 1e3
        calls_us["topk_select"] = burst_ms([functools.partial(lib.topk_select, st.scores, st.n_visible, wl.K,
                                                              L["topk"], st.ws_topk) for L in idx_layers])[0] * 1e3
        if wl.fp8_window:
            calls_us["sparse_attn_decode_fp8win"] = burst_ms([functools.partial(
                lib.sparse_attn_decode_fp8win, s.cache, L["q"], st.layers[0]["topk"], s.block_table, L["swa8"],
                L["swa8_scale"], L["swa_len"], st.scale, L["out"], L["lse"], s.ws_attn)
                for s in steps for L in st.layers])[0] * 1e3
        else:
            calls_us["sparse_attn_decode"] = burst_ms([functools.partial(
                lib.sparse_attn_decode, s.cache, L["q"], st.layers[0]["topk"], s.block_table, L["swa"], L["swa_len"],
                st.scale, L["out"], L["lse"], s.ws_attn) for s in steps for L in st.layers])[0] * 1e3
        idx_bytes = sum(int(x) for x in wl.n_entries) * IDX_ENTRY_BYTES
        tokens = wl.B
    else:
        scan = [functools.partial(lib.index_score, s.cache, s.q_idx, s.w, s.n_visible, s.block_table2d, s.scores,
                                  seq_of_query=s.seq_of_query) for s in steps]
        calls_us["topk_select"] = burst_ms([functools.partial(lib.topk_select, st.scores, st.n_visible, wl.K,
                                                              st.topk, st.ws_topk)], target=8)[0] * 1e3
        calls_us["sparse_attn_prefill_chunk"] = burst_ms([functools.partial(
            lib.sparse_attn_prefill_chunk, s.cache, st.q, st.topk, s.block_table, int(wl.ctx[0]), st.swa,
            st.swa_first_valid, wl.W, st.scale, st.out, st.lse, st.ws_attn) for s in steps], target=8)[0] * 1e3
        idx_bytes = int(wl.n_visible().astype("int64").sum()) * IDX_ENTRY_BYTES
        tokens = wl.chunk
        counted_ws = None
    idx_ms, idx_launches = burst_ms(scan)
    if counted_ws is not None:
        for ws_ in counted_ws:
            ws_.zero_()  # the counts the burst piled up
        calls_us["index_score_counted"] = idx_ms * 1e3
    else:
        calls_us["index_score"] = idx_ms * 1e3
    achieved = idx_bytes / (idx_ms * 1e-3) / 1e9
    traffic = stored_traffic(wl.name)
    step_bytes = fp4_bytes_per_step(wl)

    if args.copy_probe_mib > 0:
        # a plain copy kernel of known size (read N, write N) for counter calibration
        n = args.copy_probe_mib << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    res = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4(e2m1)+fp32",
        "data": "synthetic (seeded N(0,1) bf16 latents/keys/queries/window, U(0,1) head weights)",
        "config": {"workload": wl.name,
                   "context_tokens": wl.ctx if wl.kind == "schedule" else (int(wl.ctx[0]) if wl.B == 1
                                                                          else list(wl.ctx)),
                   "entries_per_seq": ([int(wl.cache_workload(w).n_entries[0]) for w in wl.writers()]
                                       if wl.kind == "schedule" else [int(x) for x in wl.n_entries][:4]),
                   "batch": wl.B, "heads": wl.H, "index_heads": wl.Hi, "topk": wl.K, "window": wl.W,
                   "layers": (",".join(wl.layers) if wl.kind in ("decode", "schedule")
                              else f"prefill chunk {wl.chunk}"),
                   "hip_graph": bool(args.graph), "cache_copies_rotated": R,
                   "touched_bytes_per_copy_step": touched},
        "cold_step_distribution": dist,
        "warm_ms_per_step": warm_ms,
        "warm_tokens_per_s": tokens / (warm_ms * 1e-3),
        "fp4_bytes_per_step": step_bytes,
        "fp4_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "fp4_frac_of_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        # the scan kernel of the indexer stage as the step runs it (with the selection's
        # digit counting: index_score_counted launches the kernel index_topk launches);
        # in decode, bursts go layer-major over the cache copies, so every launch reads
        # keys that are out of the MALL
        "roofline": {"kernel": f"index_score_kernel<{wl.Hi // 16}, 1, true, false, false>" if wl.kind != "prefill"
                     else f"index_score_q2_kernel<{wl.Hi // 16}>",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_kind": "L2-miss (fabric) bytes per launch from FETCH_SIZE + WRITE_SIZE; MALL hits "
                                     "count as misses",
                     "bytes_per_launch": idx_bytes, "avg_launch_ms": idx_ms,
                     "launches_timed": idx_launches, "cold": wl.kind != "prefill" and R > 1},
        "calls_us": calls_us,
    }
    if wl.kind == "prefill":
        # the prefill scan is a dense FP4 contraction (every query against every visible
        # key, all index heads): its roofline is the FP4 MFMA peak, not HBM
        flop = int(wl.n_visible().astype("int64").sum()) * wl.Hi * INDEX_DIM * 2
        tflops = flop / (idx_ms * 1e-3) / 1e12
        res["roofline"] = {"kernel": f"index_score_q2_kernel<{wl.Hi // 16}>", "bound": "mfma", "achieved": tflops,
                           "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / MFMA_FP4_PEAK_TFLOPS,
                           "traffic": traffic, "flop_per_launch": flop, "avg_launch_ms": idx_ms,
                           "launches_timed": idx_launches}
        res["roofline_hbm_view"] = {"kernel": "index_score", "achieved": achieved, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "bytes_per_launch": idx_bytes}
        # attention: q.k over the selected entries and the window, then p.v, all heads
        # (bf16 MFMA after dequantisation)
        attn_flop = wl.chunk * (wl.K + wl.W) * wl.H * LATENT_DIM * 2 * 2
        attn_ms = calls_us["sparse_attn_prefill_chunk"] * 1e-3
        res["attention_mfma_bf16"] = {"kernel": "sparse_attn_prefill_chunk",
                                      "achieved": attn_flop / (attn_ms * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                                      "unit": "TFLOP/s",
                                      "frac": attn_flop / (attn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                      "flop_per_launch": attn_flop}
    if not args.no_cpu_baseline:
        import oracle  # the CPU baseline leg only

        oracle.set_num_threads(args.cpu_threads)
        res["cpu_baseline"] = cpu_baseline(wl)
        res["cpu_baseline"]["cpu_model"] = cpu_model()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
