#!/usr/bin/env python3
"""Benchmark of one decode step of one hybrid-sparse-attention layer at 1M context on MI355X.

Headline workload (synthetic, seeded; the pages measure on no public dataset): a C4 layer, bf16
storage with fp32 arithmetic, one sequence of 1,048,576 tokens, groups of m = 4, so 262,144
compressed entries and index candidates; top-512; a 128-token window; 64 query heads over a
512-wide shared latent; indexer 4 heads x 128.

One step = one decode step of the layer, the whole decode path of the hot path over inputs already
resident in device memory: chs_decode_step (indexer scores over the 262,144 candidates, the exact
top-512, one softmax over the 128 window rows and the 512 selected entries). The K timed steps are
one replay of a HIP graph that captures K steps; every step reads one of C rotated input sets
(index keys, indexer query and weights, query, window), each set selecting its own 512 entries, so
the 64 MiB key scan and the gathers read cold data (C x 64 MiB of keys exceeds the 256 MB Infinity
Cache). `value` is the median step time over repeated replays of that graph; `ms_per_step` is the
timed replay's wall clock divided by K. The prefill compression that fills the cache is timed on
its own (a component), not folded into the step.

`roofline` describes the step's dominant kernel, the index-score kernel (score_mfma_kernel, about
40% of the step): its algorithmic bytes (the keys, the indexer query and weights, read once) over
its average launch duration, taken with HIP events around chs_index_scores on the stream it runs
on; `traffic` is its FETCH_SIZE + WRITE_SIZE per launch from the committed counter summary, scaled
by a plain copy's counters, when that summary was taken on the current kernel sources.

Components (each with its algorithmic bytes and fraction of the 8 TB/s HBM roofline): every
compressor run of the five workloads (m = 4 and m = 128), the C4 step at 128K (batch 1) and at
200K x 64 sequences, the C128 step at 4 x 1M and at 200K x 64, the standalone top-512 of 262,144
(one row and 64 rows), the step as two calls, the step over FP8 storage (one call and two), the per-token step with
appends, the step over paged pools (one call and two), the working-set gather and the batched appends. `cpu_baseline`
is the CPU oracle timed on this host on a bounded sample (a reported baseline, not a target).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn-layer µs/step at 1M ctx; top-512-of-256K µs; compressor HBM GB/s"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_c4_1m_bf16_traffic.txt")
CSRC = os.path.join(ROOT, "compressed_hybrid_sparse_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=8, help="rotated decode input sets (64 MiB of keys each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the components (profiling runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (known bytes) for counter scaling")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_hash):
    """HBM bytes per launch of the score kernel from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line and ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def median(xs):
    return statistics.median(xs) if xs else float("nan")


def frac(nbytes, us):
    return None if not us else round(nbytes / (us * 1e-6) / (HBM_PEAK_GBPS * 1e9), 4)


def r2(x):
    return None if x is None else round(x, 2)


# ------------------------------------------------------------------ algorithmic bytes
# Inputs read once plus outputs written once; implementation traffic (the fp32 score round trip,
# group statistics, split partials, re-reads) is excluded and shows up in the counters.
def compress_bytes(groups, m, d, e=2):
    ng = int(sum(int(g) for g in groups))
    return 2 * ng * m * d * e + m * d * 4 + ng * d * e


def c4_step_bytes(groups, swa, k, H, d, Hi, dI, e=2):
    tot = 0
    for G, s in zip(groups, swa):
        G, s = int(G), int(s)
        tot += G * dI * e + Hi * dI * e + Hi * 4 + k * 4 + (min(k, G) + s) * d * e + H * d * e + H * d * 4 + H * 4
    return tot


def c128_step_bytes(groups, swa, H, d, e=2):
    return int(sum((int(G) + int(s)) * d * e + H * d * e + H * d * 4 + H * 4 for G, s in zip(groups, swa)))


# ------------------------------------------------------------------ timing helpers
def make_timers(torch):
    def events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    # A spin kernel holds the stream while the host enqueues the timed calls, so that no host-side
    # gap (argument checks, launch) falls between an event and the call it brackets.
    torch.cuda._sleep(1 << 10)                  # the spin kernel's first launch loads its code
    torch.cuda.synchronize()
    a, b = events(1)[0]
    torch.cuda._sleep(1 << 16)                  # the GPU is busy before the calibrated interval begins
    a.record()
    torch.cuda._sleep(1 << 22)
    b.record()
    torch.cuda.synchronize()
    cycles_per_us = (1 << 22) / max(a.elapsed_time(b) * 1e3, 1e-3)

    def per_call_us(fn, reps, warm=3):
        """Events around each call on the current stream (stream launches, the queue kept full)."""
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn(warm)
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        ev = events(reps)
        hold = events(1)[0]
        hold[0].record()
        torch.cuda._sleep(int(cycles_per_us * (3 * reps * host_us + 2000)))
        hold[1].record()
        t0 = time.perf_counter()
        for i in range(reps):
            ev[i][0].record()
            fn(warm + 1 + i)
            ev[i][1].record()
        enq_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        if hold[0].elapsed_time(hold[1]) * 1e3 < enq_us:
            log(f"note: the host enqueue ({enq_us:.0f} us) outlasted the hold; the first intervals may include "
                "host gaps")
        return [x.elapsed_time(y) * 1e3 for x, y in ev]

    def burst_us(fn, reps, warm=3):
        """Average time of `reps` calls launched back to back between two events, the queue kept full
        (no event between the calls, so this is the launches' average duration plus the dispatch gap
        between consecutive kernels)."""
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn(warm)
        host_us = (time.perf_counter() - t0) * 1e6
        torch.cuda.synchronize()
        a_, b_ = events(1)[0]
        torch.cuda._sleep(int(cycles_per_us * (3 * reps * host_us + 2000)))
        a_.record()
        for i in range(reps):
            fn(warm + 1 + i)
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) * 1e3 / reps

    def graph(fn, count):
        """A HIP graph of fn(0) .. fn(count - 1), replayed once (untimed) before it is returned."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        return g

    def graph_us(fn, count, reps=20):
        """Median per-call time of `count` calls replayed back to back from one graph."""
        try:
            g = graph(fn, count)
        except Exception as exc:   # an extra measurement: say why it is missing
            log(f"graph replay unavailable: {exc}")
            return None
        ev = events(reps)
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        return median([a.elapsed_time(b) * 1e3 / count for a, b in ev])

    return per_call_us, burst_us, graph, graph_us


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(wl, layer):
    """The CPU oracle's own decode step on the headline workload's inputs, timed on the host cores:
    index scores over all 262,144 candidates, full-sort top-512, the compression of the 512 selected
    groups and the attention over 128 + 512 keys. Input regeneration is not timed."""
    import numpy as np

    import oracle
    from synth import workloads as W
    n = wl.lengths[0]
    G = n // layer.m
    q, qi, w = W.host_q(wl, layer)[0], W.host_qidx(wl, layer)[0], W.host_w(wl, layer)[0]
    K = W.host_index_keys(wl, layer, 0, 0, G)
    win = W.host_tokens(wl, layer, W.T_X, 0, n - wl.window, n)
    bias = W.host_bias(wl, layer)
    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        s = oracle.index_scores(qi, w, K).astype(np.float32)
        sel = oracle.topk(s, layer.k)
        t1 = time.perf_counter()
        groups = sel[sel >= 0]
        X = np.concatenate([W.host_tokens(wl, layer, W.T_X, 0, g * layer.m, (g + 1) * layer.m) for g in groups])
        Z = np.concatenate([W.host_tokens(wl, layer, W.T_Z, 0, g * layer.m, (g + 1) * layer.m) for g in groups])
        t2 = time.perf_counter()
        C = oracle.store(oracle.compress(X, Z, bias, layer.m, [0, X.shape[0]]), True)
        oracle.attend(q, oracle.step_keys(win, C, None), wl.d ** -0.5)
        t3 = time.perf_counter()
        times.append((t1 - t0) + (t3 - t2))
    # Compressor: the first 65,536 tokens (1/16 of the prefill), scaled to the full prefill.
    sample = 65536
    Xs = W.host_tokens(wl, layer, W.T_X, 0, 0, sample)
    Zs = W.host_tokens(wl, layer, W.T_Z, 0, 0, sample)
    t0 = time.perf_counter()
    oracle.compress(Xs, Zs, bias, layer.m, [0, sample])
    tc = (time.perf_counter() - t0) * (n / sample)
    return {
        "value": round(median(times) * 1e6, 1),
        "unit": "µs/step",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": ("the oracle's full decode step on the headline inputs (scores of all 262144 candidates, "
                   "full-sort top-512, compression of the 512 selected groups, attention over 640 keys), "
                   "median of 5; compress_us_scaled: the oracle compressor on the first 65536 tokens "
                   "scaled x16 to the 1M-token prefill"),
        "compress_us_scaled": round(tc * 1e6, 1),
        "host_cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ decode input sets
def decode_sets(torch, synth, W, wl, layer, inp, copies, dev):
    """`copies` input sets for the decode step: set 0 is the workload's own (index keys, indexer query
    and weights, query, window); set i > 0 has its own indexer query, weights, query and window, drawn
    from the same generator streams further along, and its own copy of the keys, so every set selects
    its own entries and reads its own 64 MiB of keys."""
    dt = torch.bfloat16
    tb = layer.tensor_base
    sets = [dict(keys=inp["k_idx"], q_idx=inp["q_idx"], w=inp["w"], q=inp["q"], swa=inp["swa_kv"])]
    for i in range(1, copies):
        off = i << 24
        s = dict(keys=inp["k_idx"].clone())
        s["q_idx"] = synth.gpu_normal(torch.empty_like(inp["q_idx"]), wl.seed, tb + W.T_QI, off)
        s["w"] = synth.gpu_uniform(torch.empty_like(inp["w"]), wl.seed, tb + W.T_W, off)
        s["q"] = synth.gpu_normal(torch.empty_like(inp["q"]), wl.seed, tb + W.T_Q, off)
        s["swa"] = synth.gpu_normal(torch.empty_like(inp["swa_kv"]), wl.seed, tb + W.T_X, off)
        sets.append(s)
    return sets


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU "
              f"leg (asked for --gpus {args.gpus}). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import compressed_hybrid_sparse_amd as chs
    import synth
    from synth import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    per_call_us, burst_us, make_graph, graph_us = make_timers(torch)
    comps = {}

    # ---------------------------------------------------------------- headline workload inputs
    wl = W.workload(4)
    layer = wl.layers[0]
    n, d, H, k = wl.lengths[0], wl.d, wl.heads, layer.k
    G = n // layer.m
    scale = d ** -0.5
    log(f"inputs: {wl.name}")
    inp = W.device_inputs(wl, layer, dev)
    comp = torch.empty(G, d, dtype=torch.bfloat16, device=dev)

    def compress4(_i):
        chs.compress(inp["X"], inp["Z"], inp["bias"], layer.m, inp["cu_tokens"], inp["cu_groups"], G, comp)

    c4_us = per_call_us(compress4, 5, warm=2)
    comps["compress_c4_1m_bf16"] = dict(m=4, tokens=n, median_us=r2(median(c4_us)),
                                        algorithmic_bytes=compress_bytes([G], 4, d),
                                        hbm_frac=frac(compress_bytes([G], 4, d), median(c4_us)),
                                        value_source="events around each call")
    # The same prefill with E4M3 output (chs_compress_fp8): the FP8 step below reads these entries.
    comp8 = torch.empty(G, d, dtype=torch.uint8, device=dev)
    comp8_s = torch.empty(G, dtype=torch.float32, device=dev)

    def compress4_fp8(_i):
        chs.compress_fp8(inp["X"], inp["Z"], inp["bias"], layer.m, inp["cu_tokens"], inp["cu_groups"], G, comp8,
                         comp8_s)

    c8_us = per_call_us(compress4_fp8, 5, warm=2)
    c8_bytes = compress_bytes([G], 4, d) - G * d * 2 + G * (d + 4)
    comps["compress_fp8_c4_1m_bf16"] = dict(call="chs_compress_fp8", m=4, tokens=n, median_us=r2(median(c8_us)),
                                            algorithmic_bytes=c8_bytes, hbm_frac=frac(c8_bytes, median(c8_us)))
    del inp["X"], inp["Z"]
    torch.cuda.empty_cache()

    sets = decode_sets(torch, synth, W, wl, layer, inp, args.copies, dev)
    C = len(sets)
    scores = torch.empty(G, dtype=torch.float32, device=dev)
    topk = torch.empty(1, k, dtype=torch.int32, device=dev)
    out = torch.empty(1, H, d, dtype=torch.float32, device=dev)
    lse = torch.empty(1, H, dtype=torch.float32, device=dev)
    cu = inp["cu_groups"]
    swa_len = inp["swa_len"]
    ws_step = chs.decode_step_workspace(1, H, d, wl.window, k, G, dev)

    def step(i):
        s = sets[i % C]
        chs.decode_step(s["q_idx"], s["w"], s["keys"], s["q"], s["swa"], swa_len, comp, cu, k, scale, G, scores,
                        ws_step, topk, out, lse)

    # ---------------------------------------------------------------- the timed steps
    log(f"headline: {args.warmup} warmup steps, then {args.steps} steps in one graph replay")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    g_steps = make_graph(step, args.steps)      # capture, one untimed replay
    torch.cuda.synchronize()                    # barrier (one rank) + sync on both sides
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in ev:
        a.record()
        g_steps.replay()
        b.record()
    torch.cuda.synchronize()
    step_us = median([a.elapsed_time(b) * 1e3 / args.steps for a, b in ev])
    stream_us = median(per_call_us(step, 4 * C))
    del g_steps
    step_bytes = c4_step_bytes([G], [wl.window], k, H, d, wl.idx_heads, wl.idx_dim)

    # ---------------------------------------------------------------- the dominant kernel
    ws_sc = chs.index_topk_workspace(1, G, 1, dev)

    def scores_only(i):
        s = sets[i % C]
        chs.index_scores(s["q_idx"], s["w"], s["keys"], cu, G, scores, ws_sc)

    sc_us_list = per_call_us(scores_only, 8 * C)
    sc_us = burst_us(scores_only, 8 * C)                # average launch duration, as rocprofv3 reports
    sc_bytes = G * wl.idx_dim * 2 + wl.idx_heads * wl.idx_dim * 2 + wl.idx_heads * 4
    sc_graph_us = graph_us(scores_only, C)
    kernel_hash = source_hash("index_topk.hip", "attn_core.h", "common.h")
    comps["index_scores_us"] = dict(call="chs_index_scores (score_mfma_kernel alone)",
                                    avg_us=r2(sc_us), avg_source="64 launches back to back between two events",
                                    per_call_median_us=r2(median(sc_us_list)), graph_median=r2(sc_graph_us),
                                    algorithmic_bytes=sc_bytes, hbm_frac=frac(sc_bytes, sc_us))
    comps["decode_step_fused_us"] = dict(call="chs_decode_step", value_source="graph replay, rotated input sets",
                                         graph_median=r2(step_us), stream_median=r2(stream_us),
                                         algorithmic_bytes=step_bytes, hbm_frac=frac(step_bytes, step_us))
    if not args.headline_only:
        run_components(torch, chs, synth, W, dev, comps, per_call_us, graph_us, wl, layer, inp, sets, comp, scores,
                       topk, out, lse, ws_step, step, comp8, comp8_s)
    if args.calib_copy:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()
        del a, bcopy

    result = {
        "metric": METRIC,
        "value": round(step_us, 2),
        "value_source": f"chs_decode_step (index scores + top-k + attention), median per step over 20 replays of a "
                        f"HIP graph of {args.steps} steps over {C} rotated input sets",
        "unit": "µs/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; no dataset)",
        "config": {"workload": wl.name, "batch": 1, "context_tokens": n, "m": layer.m, "candidates": G,
                   "topk": k, "window": wl.window, "heads": H, "d": d,
                   "indexer": f"{wl.idx_heads}x{wl.idx_dim}", "input_sets": C},
        "components": comps,
        "roofline": {"bound": "hbm",
                     "kernel": "score_mfma_kernel<bf16, 128, 1> (the step's index scores over 262,144 candidates; "
                               "the step's dominant kernel)",
                     "achieved": round(sc_bytes / (sc_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": frac(sc_bytes, sc_us), "traffic": read_traffic(kernel_hash),
                     "algorithmic_bytes_per_launch": sc_bytes, "avg_launch_us": r2(sc_us),
                     "step_algorithmic_bytes": step_bytes, "step_frac": frac(step_bytes, step_us),
                     "kernel_share_of_step": round(sc_us / step_us, 3),
                     "kernel_source_sha256_16": kernel_hash},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(wl, layer)
    print(json.dumps(result, default=int), flush=True)


def run_components(torch, chs, synth, W, dev, comps, per_call_us, graph_us, wl, layer, inp, sets, comp, scores, topk,
                   out, lse, ws_step, step, comp8, comp8_s):
    import numpy as np
    n, d, H, k = wl.lengths[0], wl.d, wl.heads, layer.k
    G = n // layer.m
    C = len(sets)
    scale = d ** -0.5
    cu, swa_len = inp["cu_groups"], inp["swa_len"]
    step_bytes = c4_step_bytes([G], [wl.window], k, H, d, wl.idx_heads, wl.idx_dim)

    # ---- the same step as two calls, and with hot caches (one input set replayed)
    log("components: two calls, hot step")
    ws_topk = chs.index_topk_workspace(1, G, k, dev)
    ws_attn = chs.decode_attn_workspace(torch.bfloat16, 1, H, d, wl.window, k, G, dev)

    def two_calls(i):
        s = sets[i % C]
        chs.index_topk(s["q_idx"], s["w"], s["keys"], cu, k, G, scores, ws_topk, topk)
        chs.decode_attn(s["q"], s["swa"], swa_len, comp, cu, topk, scale, G, ws_attn, out, lse)

    two_us = graph_us(two_calls, C)
    sel_us = per_call_us(lambda i: chs.index_topk(sets[i % C]["q_idx"], sets[i % C]["w"], sets[i % C]["keys"], cu, k,
                                                  G, scores, ws_topk, topk), 2 * C)
    att_us = per_call_us(lambda i: chs.decode_attn(sets[i % C]["q"], sets[i % C]["swa"], swa_len, comp, cu, topk,
                                                   scale, G, ws_attn, out, lse), 2 * C)
    hot_us = graph_us(lambda i: step(0), C)
    comps["decode_step_us"] = dict(call="chs_index_topk + chs_decode_attn", value_source="graph replay",
                                   graph_median=r2(two_us), index_topk_us=r2(median(sel_us)),
                                   decode_attn_us=r2(median(att_us)), algorithmic_bytes=step_bytes,
                                   hbm_frac=frac(step_bytes, two_us))
    comps["decode_step_hot_us"] = dict(call="chs_decode_step on one input set (keys and gathers cache-resident)",
                                       graph_median=r2(hot_us), hbm_frac_if_cold=frac(step_bytes, hot_us))

    # ---- FP8 storage written by the library: the entries by chs_compress_fp8 (in main), the index keys
    # and the windows by chs_quantize_e4m3 (E4M3 codes, one fp32 scale per row)
    log("components: fp8 step")
    fp8 = [chs.quantize_e4m3(sets[i]["keys"]) for i in range(C)]
    sw8 = [chs.quantize_e4m3(sets[i]["swa"].reshape(-1, d)) for i in range(C)]
    kq_us = per_call_us(lambda i: chs.quantize_e4m3(sets[i % C]["keys"], *fp8[i % C]), 2 * C)
    kq_bytes = G * wl.idx_dim * 2 + G * wl.idx_dim + G * 4
    comps["quantize_e4m3_keys_us"] = dict(call="chs_quantize_e4m3 (262,144 index keys of 128)",
                                          median_us=r2(median(kq_us)), algorithmic_bytes=kq_bytes,
                                          hbm_frac=frac(kq_bytes, median(kq_us)))

    def decode_fp8(i):
        codes, sc = fp8[i % C]
        s8, s8s = sw8[i % C]
        s = sets[i % C]
        chs.index_topk_fp8(s["q_idx"], s["w"], codes, sc, cu, k, G, scores, ws_topk, topk)
        chs.decode_attn_fp8(s["q"], s8.view(1, -1, d), s8s.view(1, -1), swa_len, comp8, comp8_s, cu, topk, scale, G,
                            ws_attn, out, lse)

    def decode_fp8_fused(i):
        codes, sc = fp8[i % C]
        s8, s8s = sw8[i % C]
        s = sets[i % C]
        chs.decode_step_fp8(s["q_idx"], s["w"], codes, sc, s["q"], s8.view(1, -1, d), s8s.view(1, -1), swa_len, comp8,
                            comp8_s, cu, k, scale, G, scores, ws_step, topk, out, lse)

    fp8_us = graph_us(decode_fp8, C)
    fp8_fused_us = graph_us(decode_fp8_fused, C)
    fp8_bytes = (step_bytes - G * wl.idx_dim * 2 + G * wl.idx_dim + G * 4 - (k + wl.window) * d * 2
                 + (k + wl.window) * (d + 4))
    comps["decode_step_fp8_us"] = dict(call="chs_decode_step_fp8", graph_median=r2(fp8_fused_us),
                                       two_calls="chs_index_topk_fp8 + chs_decode_attn_fp8",
                                       two_calls_graph_median=r2(fp8_us), algorithmic_bytes=fp8_bytes,
                                       hbm_frac=frac(fp8_bytes, fp8_fused_us))
    del fp8, sw8
    torch.cuda.empty_cache()

    # ---- the per-token step: appends of the new token's KV row and index key (one launch), then the
    # top-k and the attention over the grown context. Counters advance in place; comp_count feeds cu.
    log("components: per-token step with appends")
    G0 = G - 64
    cu_app = torch.tensor([0, G0], dtype=torch.int64, device=dev)
    n_kv = torch.tensor([G0 * layer.m], dtype=torch.int64, device=dev)
    n_ix = n_kv.clone()
    swa_app = inp["swa_kv"].clone()
    swa_len_app = torch.empty(1, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev).manual_seed(5)
    x_tok = torch.randn(1, d, generator=g, device=dev).bfloat16()
    z_tok = torch.randn(1, d, generator=g, device=dev).bfloat16()
    ring_kv = torch.randn(8, d, generator=g, device=dev).bfloat16()
    xi_tok = torch.randn(1, wl.idx_dim, generator=g, device=dev).bfloat16()
    zi_tok = torch.randn(1, wl.idx_dim, generator=g, device=dev).bfloat16()
    bias_i = torch.zeros(layer.m, wl.idx_dim, dtype=torch.float32, device=dev)
    swa_i = torch.randn(1, 8, wl.idx_dim, generator=g, device=dev).bfloat16()
    ring_i = torch.randn(8, wl.idx_dim, generator=g, device=dev).bfloat16()
    page0 = torch.zeros(1, dtype=torch.int32, device=dev)
    start0 = torch.zeros(1, dtype=torch.int64, device=dev)
    kv_stream = chs.append_stream(x_tok, z_tok, inp["bias"], n_kv, swa_app, ring_kv, comp, ring_page=page0,
                                  comp_start=start0, ring_size=8, swa_len=swa_len_app, comp_count=cu_app[1:])
    ix_streams = [chs.append_stream(xi_tok, zi_tok, bias_i, n_ix, swa_i, ring_i, s["keys"], ring_page=page0,
                                    comp_start=start0, ring_size=8) for s in sets]

    def decode_append(i):
        s = sets[i % C]
        chs.append_multi(layer.m, [kv_stream, ix_streams[i % C]])
        chs.index_topk(s["q_idx"], s["w"], s["keys"], cu_app, k, G, scores, ws_topk, topk)
        chs.decode_attn(s["q"], swa_app, swa_len_app, comp, cu_app, topk, scale, G, ws_attn, out, lse)

    app_step_us = graph_us(decode_append, C)
    comps["decode_step_with_append_us"] = dict(
        call="chs_append_multi (KV row + index key, one launch) + chs_index_topk + chs_decode_attn",
        graph_median=r2(app_step_us), tokens_appended=int(n_kv.item()) - G0 * layer.m)

    # ---- chs_append alone on 64 sequences (C4: ring 8, a quarter complete a group per token; C128: ring
    # 128, offsets spread over a group so one sequence pools 128 rows every other token)
    e_sz = 2

    def append_batch(mm, ring):
        Bn = 64
        cap = 4096 // mm + 64
        st = dict(n=torch.tensor([4096 + (b * mm // Bn) % mm for b in range(Bn)], dtype=torch.int64, device=dev),
                  swa=torch.randn(Bn, wl.window, d, generator=g, device=dev).bfloat16(),
                  ring=torch.randn(Bn * ring, d, generator=g, device=dev).bfloat16(),
                  page=torch.arange(Bn, dtype=torch.int32, device=dev),
                  comp=torch.empty(Bn * cap, d, dtype=torch.bfloat16, device=dev),
                  start=torch.arange(0, Bn * cap, cap, dtype=torch.int64, device=dev),
                  x=torch.randn(Bn, d, generator=g, device=dev).bfloat16(),
                  z=torch.randn(Bn, d, generator=g, device=dev).bfloat16(),
                  bias=torch.randn(mm, d, generator=g, device=dev) * 0.1,
                  sl=torch.empty(Bn, dtype=torch.int32, device=dev),
                  cc=torch.empty(Bn, dtype=torch.int64, device=dev))

        def one(i):
            chs.append(st["x"], st["z"], st["bias"], mm, st["n"], st["swa"], st["ring"], st["page"], st["comp"],
                       st["start"], ring_size=ring, swa_len=st["sl"], comp_count=st["cc"])

        us = graph_us(one, 8)
        per_group = 2 * (mm - 1) * d * e_sz + mm * d * 4 + d * e_sz
        return us, int(Bn * 4 * d * e_sz + (Bn / mm) * per_group)

    app4_us, app4_bytes = append_batch(4, 8)
    app128_us, app128_bytes = append_batch(128, 128)
    comps["append_us"] = dict(value_source="graph replay, per token", batch=64, d=d, c4_median=r2(app4_us),
                              c4_algorithmic_bytes=app4_bytes, c128_median=r2(app128_us),
                              c128_algorithmic_bytes=app128_bytes)

    # ---- paged pools: index keys and entries in 64-row pages through a permuted page table
    log("components: paged step, gather")
    PG = 64
    perm = torch.randperm(G // PG, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    pt_paged = perm[None, :].contiguous().to(dev)
    len_paged = torch.tensor([G], dtype=torch.int64, device=dev)
    swa_page0 = torch.zeros(1, dtype=torch.int32, device=dev)
    scores2d = scores.view(1, G)

    def decode_paged(i):
        s = sets[i % C]
        chs.index_topk_paged(s["q_idx"], s["w"], s["keys"], PG, pt_paged, len_paged, k, G, scores2d, ws_topk, topk)
        chs.decode_attn_paged(s["q"], s["swa"], swa_page0, swa_len, comp, PG, pt_paged, len_paged, topk, scale, G,
                              ws_attn, out, lse)

    def decode_paged_fused(i):
        s = sets[i % C]
        chs.decode_step_paged(s["q_idx"], s["w"], s["keys"], s["q"], s["swa"], swa_page0, swa_len, comp, PG, pt_paged,
                              len_paged, k, G, scale, scores2d, ws_step, topk, out, lse)

    paged_us = graph_us(decode_paged, C)
    paged_fused_us = graph_us(decode_paged_fused, C)
    comps["decode_step_paged_us"] = dict(call="chs_decode_step_paged", page_rows=PG, graph_median=r2(paged_fused_us),
                                         two_calls="chs_index_topk_paged + chs_decode_attn_paged",
                                         two_calls_graph_median=r2(paged_us),
                                         hbm_frac=frac(step_bytes, paged_fused_us))

    # ---- working-set gather of the 512 selected entries from a mirror in HBM or in pinned host memory
    work_rows = torch.empty(k, d, dtype=torch.bfloat16, device=dev)
    work_tk = torch.empty(1, k, dtype=torch.int32, device=dev)
    s0 = sets[0]
    chs.index_topk(s0["q_idx"], s0["w"], s0["keys"], cu, k, G, scores, ws_topk, topk)
    host_mirror = torch.empty(G, d, dtype=torch.bfloat16, pin_memory=True)
    host_mirror.copy_(comp)
    cu_ws = torch.tensor([0, k], dtype=torch.int64, device=dev)
    gdev = graph_us(lambda i: chs.gather_selected(comp, cu, topk, work=work_rows, work_topk=work_tk, cu_work=cu_ws), 8)
    ghost = graph_us(lambda i: chs.gather_selected(host_mirror, cu, topk, work=work_rows, work_topk=work_tk,
                                                   cu_work=cu_ws), 8)
    comps["gather_selected_us"] = dict(value_source="graph replay", rows=k, row_bytes=d * 2, from_hbm_median=r2(gdev),
                                       from_pinned_host_median=r2(ghost),
                                       host_GBps=None if not ghost else round(k * d * 2 / (ghost * 1e-6) / 1e9, 2))
    del host_mirror

    # ---- standalone top-512 of 262,144: one row (rotated over 256 copies) and 64 rows (8 copies)
    log("components: standalone top-k")
    row = torch.from_numpy(W.topk_scores(wl, "normal")).to(dev)
    rows1 = row.repeat(256)
    cu1 = torch.tensor([0, G], dtype=torch.int64, device=dev)
    ws1 = chs.index_topk_workspace(1, G, 512, dev)
    tk1 = torch.empty(1, 512, dtype=torch.int32, device=dev)
    rows64 = row.repeat(64 * 8)
    cu64 = torch.arange(0, 65 * G, G, dtype=torch.int64, device=dev)
    ws64 = chs.index_topk_workspace(64, G, 512, dev)
    tk64 = torch.empty(64, 512, dtype=torch.int32, device=dev)
    one_row = lambda i: chs.topk_from_scores(rows1[(i % 256) * G:(i % 256 + 1) * G], cu1, 512, G, ws1, tk1)  # noqa
    rows_64 = lambda i: chs.topk_from_scores(rows64[(i % 8) * 64 * G:(i % 8 + 1) * 64 * G], cu64, 512, G, ws64,  # noqa
                                             tk64)
    t1 = per_call_us(one_row, 100, warm=5)
    t64 = per_call_us(rows_64, 50, warm=5)
    t1g = graph_us(one_row, 16)
    t64g = graph_us(rows_64, 8)
    row_bytes = G * 4 + 512 * 4
    comps["topk_512_of_262144_us"] = dict(
        value_source="stream launch (events around each call); graph replay beside",
        bs1_median=r2(median(t1)), bs1_graph_median=r2(t1g), rows64_median=r2(median(t64)),
        rows64_graph_median=r2(t64g), rows64_algorithmic_bytes=64 * row_bytes,
        rows64_hbm_frac=frac(64 * row_bytes, median(t64)), rows64_graph_hbm_frac=frac(64 * row_bytes, t64g))
    del rows1, rows64
    torch.cuda.empty_cache()

    # ---- the other workloads: every compressor run, the C4 and C128 steps of workloads 2, 3 and 5
    other_workloads(torch, chs, synth, W, dev, comps, per_call_us, graph_us)


def other_workloads(torch, chs, synth, W, dev, comps, per_call_us, graph_us):
    bf = torch.bfloat16
    # ---- c4_128k_bf16: 131,072 tokens, batch 1, C4
    wl2 = W.workload(2)
    L2 = wl2.layers[0]
    log(f"components: {wl2.name}")
    inp = W.device_inputs(wl2, L2, dev)
    G2 = wl2.lengths[0] // L2.m
    comp2 = torch.empty(G2, wl2.d, dtype=bf, device=dev)
    us = per_call_us(lambda i: chs.compress(inp["X"], inp["Z"], inp["bias"], L2.m, inp["cu_tokens"], inp["cu_groups"],
                                            G2, comp2), 20, warm=3)
    cb = compress_bytes([G2], L2.m, wl2.d)
    comps["compress_c4_128k_bf16"] = dict(m=L2.m, tokens=wl2.lengths[0], median_us=r2(median(us)),
                                          algorithmic_bytes=cb, hbm_frac=frac(cb, median(us)))
    del inp["X"], inp["Z"]
    # 40 rotated input sets (8 MiB of keys and 32 MiB of entries each: 1.6 GB in all)
    nset = 40
    sets2 = []
    for i in range(nset):
        off = i << 24
        if i == 0:
            s = dict(keys=inp["k_idx"], comp=comp2, q_idx=inp["q_idx"], w=inp["w"], q=inp["q"], swa=inp["swa_kv"])
        else:
            s = dict(keys=inp["k_idx"].clone(), comp=comp2.clone(),
                     q_idx=synth.gpu_normal(torch.empty_like(inp["q_idx"]), wl2.seed, W.T_QI, off),
                     w=synth.gpu_uniform(torch.empty_like(inp["w"]), wl2.seed, W.T_W, off),
                     q=synth.gpu_normal(torch.empty_like(inp["q"]), wl2.seed, W.T_Q, off),
                     swa=synth.gpu_normal(torch.empty_like(inp["swa_kv"]), wl2.seed, W.T_X, off))
        sets2.append(s)
    H, d, k = wl2.heads, wl2.d, L2.k
    ws = chs.decode_step_workspace(1, H, d, wl2.window, k, G2, dev)
    sc = torch.empty(G2, dtype=torch.float32, device=dev)
    tk = torch.empty(1, k, dtype=torch.int32, device=dev)
    o = torch.empty(1, H, d, dtype=torch.float32, device=dev)
    ls = torch.empty(1, H, dtype=torch.float32, device=dev)

    def step2(i):
        s = sets2[i % nset]
        chs.decode_step(s["q_idx"], s["w"], s["keys"], s["q"], s["swa"], inp["swa_len"], s["comp"], inp["cu_groups"],
                        k, d ** -0.5, G2, sc, ws, tk, o, ls)

    us2 = graph_us(step2, nset)
    sb = c4_step_bytes([G2], [wl2.window], k, H, d, wl2.idx_heads, wl2.idx_dim)
    comps["c4_step_128k_bf16_us"] = dict(call="chs_decode_step", value_source="graph replay, 40 rotated input sets",
                                         graph_median=r2(us2), algorithmic_bytes=sb, hbm_frac=frac(sb, us2))
    del sets2, inp, comp2
    torch.cuda.empty_cache()

    # ---- c128_1m_bs4_bf16: 4 x 1,048,576 tokens, C128 (m = 128): the prefill compression and the dense step
    wl3 = W.workload(3)
    L3 = wl3.layers[0]
    log(f"components: {wl3.name}")
    inp = W.device_inputs(wl3, L3, dev, with_index=False)
    grp3 = [nb // L3.m for nb in wl3.lengths]
    comp3 = torch.empty(sum(grp3), wl3.d, dtype=bf, device=dev)
    us = per_call_us(lambda i: chs.compress(inp["X"], inp["Z"], inp["bias"], L3.m, inp["cu_tokens"], inp["cu_groups"],
                                            max(grp3), comp3), 5, warm=2)
    cb = compress_bytes(grp3, L3.m, wl3.d)
    comps["compress_c128_1m_bs4_bf16"] = dict(m=L3.m, tokens=int(sum(wl3.lengths)), median_us=r2(median(us)),
                                              algorithmic_bytes=cb, hbm_frac=frac(cb, median(us)))
    del inp["X"], inp["Z"]
    torch.cuda.empty_cache()
    pools = [comp3] + [comp3.clone() for _ in range(9)]         # 10 x 32 MiB rotated
    qs = [inp["q"]] + [synth.gpu_normal(torch.empty_like(inp["q"]), wl3.seed, W.T_Q, i << 24) for i in range(1, 10)]
    H, d = wl3.heads, wl3.d
    B3 = wl3.batch
    ws3 = chs.decode_attn_workspace(bf, B3, H, d, wl3.window, 0, max(grp3), dev)
    o3 = torch.empty(B3, H, d, dtype=torch.float32, device=dev)
    l3 = torch.empty(B3, H, dtype=torch.float32, device=dev)

    def c128_3(i):
        chs.decode_attn(qs[i % 10], inp["swa_kv"], inp["swa_len"], pools[i % 10], inp["cu_groups"], None, d ** -0.5,
                        max(grp3), ws3, o3, l3)

    us3 = graph_us(c128_3, 10)
    sb = c128_step_bytes(grp3, list(wl3.swa_len()), H, d)
    comps["c128_step_1m_bs4_bf16_us"] = dict(call="chs_decode_attn (no top-k: every entry)",
                                             value_source="graph replay, 10 rotated entry pools", graph_median=r2(us3),
                                             algorithmic_bytes=sb, hbm_frac=frac(sb, us3),
                                             mfma_tflops=round(4 * H * d * sum(g + 128 for g in grp3) / (us3 * 1e-6)
                                                               / 1e12, 1) if us3 else None)
    comps["decode_c128_us"] = dict(same_as="c128_step_1m_bs4_bf16_us", graph_median=r2(us3), hbm_frac=frac(sb, us3))
    del pools, qs, inp, comp3
    torch.cuda.empty_cache()

    # ---- 64 sequences of 200,000 +-5% tokens; a C4 layer (m = 4) and a C128 layer (m = 128)
    wl5 = W.workload(5)
    for L5 in wl5.layers:
        log(f"components: {wl5.name} {L5.kind}")
        inp = W.device_inputs(wl5, L5, dev)
        grp = [nb // L5.m for nb in wl5.lengths]
        comp5 = torch.empty(sum(grp), wl5.d, dtype=bf, device=dev)
        us = per_call_us(lambda i: chs.compress(inp["X"], inp["Z"], inp["bias"], L5.m, inp["cu_tokens"],
                                                inp["cu_groups"], max(grp), comp5), 5, warm=2)
        cb = compress_bytes(grp, L5.m, wl5.d)
        comps[f"compress_{L5.kind}_bs64_200k_bf16"] = dict(m=L5.m, tokens=int(sum(wl5.lengths)), median_us=r2(median(us)),
                                                           algorithmic_bytes=cb, hbm_frac=frac(cb, median(us)))
        del inp["X"], inp["Z"]
        torch.cuda.empty_cache()
        H, d, B5 = wl5.heads, wl5.d, wl5.batch
        o5 = torch.empty(B5, H, d, dtype=torch.float32, device=dev)
        l5 = torch.empty(B5, H, dtype=torch.float32, device=dev)
        qs = [inp["q"], synth.gpu_normal(torch.empty_like(inp["q"]), wl5.seed, L5.tensor_base + W.T_Q, 1 << 24)]
        swa_l = list(wl5.swa_len())
        if L5.k is not None:
            k = L5.k
            qis = [inp["q_idx"], synth.gpu_normal(torch.empty_like(inp["q_idx"]), wl5.seed,
                                                  L5.tensor_base + W.T_QI, 1 << 24)]
            ws = chs.decode_step_workspace(B5, H, d, wl5.window, k, max(grp), dev)
            sc = torch.empty(sum(grp), dtype=torch.float32, device=dev)
            tk = torch.empty(B5, k, dtype=torch.int32, device=dev)

            def step5(i):
                chs.decode_step(qis[i % 2], inp["w"], inp["k_idx"], qs[i % 2], inp["swa_kv"], inp["swa_len"], comp5,
                                inp["cu_groups"], k, d ** -0.5, max(grp), sc, ws, tk, o5, l5)

            us5 = graph_us(step5, 4)
            sb = c4_step_bytes(grp, swa_l, k, H, d, wl5.idx_heads, wl5.idx_dim)
            comps["c4_step_bs64_200k_bf16_us"] = dict(call="chs_decode_step (64 sequences)",
                                                      value_source="graph replay (818 MB of keys per step)",
                                                      graph_median=r2(us5), algorithmic_bytes=sb,
                                                      hbm_frac=frac(sb, us5))
        else:
            pools = [comp5] + [comp5.clone() for _ in range(3)]     # 4 x 102 MB rotated
            ws = chs.decode_attn_workspace(bf, B5, H, d, wl5.window, 0, max(grp), dev)

            def c128_5(i):
                chs.decode_attn(qs[i % 2], inp["swa_kv"], inp["swa_len"], pools[i % 4], inp["cu_groups"], None,
                                d ** -0.5, max(grp), ws, o5, l5)

            us5 = graph_us(c128_5, 4)
            sb = c128_step_bytes(grp, swa_l, H, d)
            comps["c128_step_bs64_200k_bf16_us"] = dict(call="chs_decode_attn (64 sequences, every entry)",
                                                        value_source="graph replay, 4 rotated entry pools",
                                                        graph_median=r2(us5), algorithmic_bytes=sb,
                                                        hbm_frac=frac(sb, us5))
            del pools
        del inp, comp5, qs
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
