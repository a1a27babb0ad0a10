#!/usr/bin/env python3
"""Benchmark: paged split-KV GQA decode attention on one MI355X.

One step = pa_decode_run + pa_decode_combine (split-KV decode kernel + combine
kernel) over the whole batch, on one stream, with every input resident in HBM
(--fused-combine merges inside the decode kernel instead).  The plan is built once
before timing (it is reusable while lengths are unchanged) and timed separately.  Default workload: GQA decode at a Llama-70B-like shape (B=32,
Hq=64, Hkv=8, D=128, bf16 KV, 64-token pages, 4096 tokens each, balanced plan).

Prints ONE JSON line.  `value` is the achieved algorithmic KV bandwidth (GB/s) of a
whole step; `roofline` is for the dominant kernel (the decode kernel), timed with
HIP events on the launch stream over a graph of back-to-back launches (its device
time; eager launches of a small kernel time the host's launch rate instead);
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same workload.
A workload whose KV pool fits in the 256 MB last-level cache is also timed cold
(`cold`: each step reads the next of enough pool copies to exceed 512 MB), and its
roofline figure is the cold one.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# The pages' own numbers for a workload measured here: the MetaX paged GQA decode (HD64,
# Hq/Hkv 32/4, page 256, 1536 tokens, 8 splits), split-KV kernel plus combine kernel, 10
# groups of 100 calls, median of group means, graph mode (MetaX PR page, performance
# table; a 25 % compute slice of a MetaX C500).  Another machine: context, not a target.
PAGES_GRAPH_US = {(2, 1): 152.52, (2, 8): 248.43}
MFMA_BF16_PEAK_TFLOPS = 2500.0
MLA_FLOP_PER_TOKEN = 2 * 128 * (576 + 512)   # q.k over 576 dims and p.v over 512, 128 heads


def counter_traffic(workload, batch):
    """Calibrated HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings, or None when the kernel source has
    changed since they were taken (or none were taken for this workload)."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
        w = rec["workloads"]["%s, B=%d" % (workload, batch)]
        with open(os.path.join(ROOT, w["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != w["source_sha256"]:
                return None
        return int(round(w["fetch_kib"] * 1024 * rec["fetch_factor"]
                         + w["write_kib"] * 1024 * rec["write_factor"]))
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload index (default 1)")
    ap.add_argument("--batch", type=int, default=None, help="batch of the HD64 workload (1 or 8)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per request (linear speculative draft)")
    ap.add_argument("--topk", type=int, default=0,
                    help="sparse decode over topk listed positions per request (MLA workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-graph", action="store_true", help="skip timing a hipGraph replay of the step")
    ap.add_argument("--no-protocol", action="store_true",
                    help="skip the grouped timing (10 groups of 100 calls, median of group means)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip measuring the HBM read ceiling of the box")
    ap.add_argument("--cold-copies", type=int, default=-1,
                    help="also time with each step reading the next of N copies of the KV pool "
                         "(so that the pool is not cache-resident); -1: automatic (enough copies "
                         "to exceed 512 MB when one pool fits in the 256 MB last-level cache), 0: off")
    ap.add_argument("--fused-combine", action="store_true",
                    help="merge chunks inside the decode kernel (last workgroup per request) "
                         "instead of the combine kernel")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the path would "
              "shard by request or KV head with no exchange, or by sequence with an all-gather "
              "of the (O, lse) partials before the same combine kernel",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mqa_split_kv_amd import binding as pb
    from mqa_split_kv_amd import synth

    torch.cuda.set_device(0)
    t_gen = time.time()
    case = synth.config_case(args.config, B=args.batch, **({"q_len": args.q_len}
                                                           if args.q_len != 1 else {}))
    if args.topk:
        case.update(topk=args.topk, indices=synth.sparse_indices(case, args.topk, 7000 + args.config))
    gen_s = time.time() - t_gen
    print(f"[bench] generated workload {args.config} ({case['name']}) in {gen_s:.1f}s", file=sys.stderr,
          flush=True)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    q, kp = dev(case["q"]), dev(case["k_pool"])
    vp = dev(case["v_pool"]) if case.get("v_pool") is not None else None
    ks = dev(case["k_scale"]) if case.get("k_scale") is not None else None
    vs = dev(case["v_scale"]) if case.get("v_scale") is not None else None
    bt, sl = dev(case["block_table"]), dev(case["seq_lens"])
    idx = dev(case["indices"]) if args.topk else None
    B, Hq, Dv = case["B"], case["Hkv"] * case["G"], case["Dv"]
    out = torch.empty((B, args.q_len, Hq, Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, args.q_len, Hq), dtype=torch.float32, device="cuda")
    desc = pb.desc_from_case(case, fused=args.fused_combine)
    runner = pb.PagedDecode(desc)
    stream = torch.cuda.current_stream()

    # plan (once; timed separately)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    runner.plan(sl)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        runner.plan(sl)
    e1.record()
    torch.cuda.synchronize()
    plan_us = e0.elapsed_time(e1) * 1000.0 / 10

    def step():
        runner.run(q, kp, vp, bt, sl, out, lse, k_scale=ks, v_scale=vs, indices=idx)
        runner.combine(out, lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps bracketed by synchronisation
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    step_ms = ev0.elapsed_time(ev1) / args.steps

    # dominant kernel alone: the decode kernel, back to back on the same stream
    nk = max(args.steps, 50)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(nk):
        runner.run(q, kp, vp, bt, sl, out, lse, k_scale=ks, v_scale=vs, indices=idx)
    k1.record(stream)
    torch.cuda.synchronize()
    decode_us = k0.elapsed_time(k1) * 1000.0 / nk
    runner.combine(out, lse)
    torch.cuda.synchronize()

    # grouped timing (the MetaX page's protocol: 10 groups of 100 calls after the warm-ups,
    # median of the group means), eager here and from graphs below
    groups, calls = 10, 100

    def median_of_groups(one_group):
        means = []
        for _ in range(groups):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            one_group()
            a1.record(stream)
            torch.cuda.synchronize()
            means.append(a0.elapsed_time(a1) * 1000.0 / calls)
        return round(float(np.median(means)), 2)

    proto = None
    if not args.no_protocol:
        def eager_group():
            for _ in range(calls):
                step()
        proto = {"groups": groups, "calls_per_group": calls, "eager_us_median": median_of_groups(eager_group),
                 "graph_us_median": None}

    graph_us = decode_graph_us = None
    if not args.no_graph:
        # several steps per graph, so that the per-replay launch cost is amortised and
        # the figure is the device time of a step
        per_graph = 20
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                step()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // per_graph)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1000.0 / (reps * per_graph)
        if proto is not None:
            def graph_group():
                for _ in range(calls // per_graph):
                    g.replay()
            proto["graph_us_median"] = median_of_groups(graph_group)
        # the decode kernel alone, launched from a graph: its device time without the host's
        # per-launch cost (which is what eager back-to-back launches of a small kernel time)
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd):
            for _ in range(per_graph):
                runner.run(q, kp, vp, bt, sl, out, lse, k_scale=ks, v_scale=vs, indices=idx)
        gd.replay()
        torch.cuda.synchronize()
        g0.record()
        for _ in range(reps):
            gd.replay()
        g1.record()
        torch.cuda.synchronize()
        decode_graph_us = g0.elapsed_time(g1) * 1000.0 / (reps * per_graph)
        runner.combine(out, lse)
        torch.cuda.synchronize()

    cold = None
    pool_bytes = sum(t.numel() * t.element_size() for t in (kp, vp, ks, vs) if t is not None)
    ncold = args.cold_copies
    if ncold < 0:
        ncold = min(-(-(512 << 20) // pool_bytes) + 1, 1024) if pool_bytes < (256 << 20) else 0
    if ncold > 0:
        cold = cold_timing(runner, case, ncold, args, (q, kp, vp, ks, vs, bt, sl, out, lse, idx), stream)

    kv_bytes = synth.kv_bytes(case)
    io = synth.io_bytes(case)
    step_us = step_ms * 1000.0
    gbs = kv_bytes / (step_us * 1e-6) / 1e9
    # the dominant kernel's time per launch: from a graph of launches when timed (device
    # time), else from eager back-to-back launches
    kern_us = decode_us if decode_graph_us is None else decode_graph_us
    dec_gbs = kv_bytes / (kern_us * 1e-6) / 1e9
    fmt = {0: "bf16", 1: "fp8e4m3-kv/bf16", 2: "mla656-fp8/bf16"}[case["kv_format"]]

    traffic = counter_traffic(case["name"], B) if args.q_len == 1 and not args.topk else None
    if case["kv_format"] == 2:
        # MLA: 128 heads share each token, so the contraction is MFMA-bound
        kern_us = kern_us if cold is None else (cold["decode_kernel_graph_us"] or cold["decode_kernel_us"])
        tokens = kv_bytes / synth.MLA_TOKEN_BYTES      # attended keys (listed ones if sparse)
        tflops = MLA_FLOP_PER_TOKEN * args.q_len * tokens / (kern_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "kernel": "pa_mla_kernel",
                "timing": "warm, " + ("eager launches" if decode_graph_us is None else "graph of launches")}
    else:
        # a pool that fits in the last-level cache is quoted against HBM only cold
        cold_us = None if cold is None else (cold["decode_kernel_graph_us"] or cold["decode_kernel_us"])
        roof_gbs = dec_gbs if cold is None else kv_bytes / (cold_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(roof_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(roof_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "pa_decode_kernel<%d,%s>" % (case["D"], "bf16" if case["kv_format"] == 0 else "fp8"),
                "timing": ("warm" if cold is None else "cold (%d rotating pool copies)" % cold["copies"])
                          + (", eager launches" if decode_graph_us is None else ", graph of launches")}
    roof["algorithmic_bytes"] = kv_bytes

    ceiling = None
    if not args.no_read_ceiling:
        try:
            from mqa_split_kv_amd import probe
            ceiling = probe.read_ceiling(gib=1.0, reps=3, grids=(2048, 4096))["best_gbs"]
        except RuntimeError as e:                   # the probe library is not built
            print(f"[bench] read ceiling not measured: {e}", file=sys.stderr)
    if ceiling and roof["bound"] == "hbm":
        roof["frac_of_read_ceiling"] = round(roof["achieved"] / ceiling, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args.cpu_seconds)

    cfg = {"workload": case["name"], "B": B, "Hq": Hq, "Hkv": case["Hkv"], "D": case["D"],
           "Dv": Dv, "page_size": case["page_size"], "seq_len_total": int(np.sum(case["seq_lens"])),
           "kv_format": fmt, "q_len": args.q_len, "topk": args.topk or None, "num_splits": "balanced plan" if desc.num_splits == 0 else desc.num_splits,
           "num_parts": pb.pa_decode_num_parts(desc),
           "combine": "fused in the decode kernel" if args.fused_combine else "combine kernel",
           "parallelism": "single GPU"}
    # vs_baseline: only where the pages give a number for this very workload (same step, same
    # timing protocol): their graph µs per call over this run's graph median
    vs_baseline, vs_basis = None, None
    ref_us = PAGES_GRAPH_US.get((args.config, B))
    if ref_us is not None and args.q_len == 1 and not args.topk and proto and proto.get("graph_us_median"):
        vs_baseline = round(ref_us / proto["graph_us_median"], 2)
        vs_basis = (f"pages' graph us per call {ref_us} (MetaX C500, 25 % slice) / this graph median "
                    f"{proto['graph_us_median']:.2f} us; another machine, context only")
    rec = {
        "metric": "decode-attention µs/step + achieved KV HBM GB/s (% of MI355X peak)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "us_per_step": round(step_us, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs_baseline,
        "vs_baseline_basis": vs_basis,
        "dtype": "bf16" if case["kv_format"] == 0 else fmt,
        "data": "synthetic (seeded N(0,1), random page permutation)",
        "config": cfg,
        "kv_bytes_per_step": kv_bytes,
        "io_bytes_per_step": io,
        "plan_us": round(plan_us, 2),
        "decode_kernel_us": round(decode_us, 2),
        "decode_kernel_graph_us": None if decode_graph_us is None else round(decode_graph_us, 2),
        "graph_us_per_step": None if graph_us is None else round(graph_us, 2),
        "wall_s_timed": round(wall_s, 4),
        "roofline": roof,
        "cold": None if cold is None else dict(cold, kv_gbs_step=round(kv_bytes / (cold["us_per_step"] * 1e-6) / 1e9, 1),
                                               pct_of_hbm_peak_step=round(100.0 * kv_bytes / (cold["us_per_step"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)),
        "timing_protocol": proto,
        "read_ceiling_gbs": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cold_timing(runner, case, ncopies, args, bufs, stream):
    """The step, the decode kernel and a graph of steps, each step reading the next of
    `ncopies` copies of the KV pool (and scales): with more bytes than the last-level
    cache holds, every step's KV comes from HBM."""
    import torch

    q, kp, vp, ks, vs, bt, sl, out, lse, idx = bufs
    copies = [tuple(None if t is None else t.clone() for t in (kp, vp, ks, vs)) for _ in range(ncopies)]
    torch.cuda.synchronize()

    def run(i):
        k, v, a, b = copies[i % ncopies]
        runner.run(q, k, v, bt, sl, out, lse, k_scale=a, v_scale=b, indices=idx)

    def step(i):
        run(i)
        runner.combine(out, lse)

    n = max(args.steps, 2 * ncopies)
    for i in range(ncopies):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1000.0 / n
    e0.record(stream)
    for i in range(n):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1000.0 / n
    graph_us = dec_graph_us = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(ncopies):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(2, n // ncopies)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1000.0 / (reps * ncopies)
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd):
            for i in range(ncopies):
                run(i)
        gd.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            gd.replay()
        e1.record()
        torch.cuda.synchronize()
        dec_graph_us = e0.elapsed_time(e1) * 1000.0 / (reps * ncopies)
        runner.combine(out, lse)
        torch.cuda.synchronize()
    pool = sum(t.numel() * t.element_size() for t in copies[0] if t is not None)
    del copies
    torch.cuda.empty_cache()
    return {"copies": ncopies, "bytes_rotated": pool * ncopies, "us_per_step": round(step_us, 2),
            "decode_kernel_us": round(dec_us, 2), "graph_us_per_step": None if graph_us is None else round(graph_us, 2),
            "decode_kernel_graph_us": None if dec_graph_us is None else round(dec_graph_us, 2)}


def cpu_baseline(case, seconds):
    """Time the fp64 CPU oracle on a bounded sample of (request, KV head) pairs."""
    import numpy as np

    import oracle
    from mqa_split_kv_amd import synth

    B, Hkv = case["B"], case["Hkv"]
    threads = oracle.threads(0)
    L = np.asarray(case["seq_lens"], np.int64)
    if case.get("topk"):                            # keys each request attends to
        idx = np.asarray(case["indices"])
        L = ((idx >= 0) & (idx < L[:, None])).sum(axis=1).astype(np.int64)
    order = [(b, h) for b in range(B) for h in range(Hkv)]
    n = max(1, min(len(order), threads))
    spent, done_pairs, done_tokens, reps = 0.0, 0, 0, 1
    while True:
        pairs = np.zeros((B, Hkv), bool)
        sel = order[:n]
        for b, h in sel:
            pairs[b, h] = True
        t0 = time.perf_counter()
        oracle.decode(case, pairs=pairs)
        dt = time.perf_counter() - t0
        spent, done_pairs = dt, n
        done_tokens = int(sum(L[b] for b, _ in sel))
        if dt >= seconds or n == len(order):
            break
        n = min(len(order), max(n + 1, int(n * min(8.0, 1.5 * seconds / max(dt, 1e-3)))))
    # the whole workload fits in the budget: repeat it until the budget is spent
    while spent * reps < seconds and reps < 1000:
        extra = max(1, int((seconds - spent * reps) / max(spent, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(extra):
            oracle.decode(case, pairs=pairs)
        dt = time.perf_counter() - t0
        spent = (spent * reps + dt) / (reps + extra)
        reps += extra
    per_tok_head = synth.kv_bytes(case) / max(1, int(L.sum()) * Hkv)
    gbs = done_tokens * per_tok_head / spent / 1e9
    full_us = spent * 1e6 * (int(L.sum()) * Hkv) / max(1, done_tokens)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done_pairs} of {B * Hkv} (request, KV head) pairs, {done_tokens} tokens, "
                      f"{reps} run(s), {spent:.2f} s each; full step extrapolates to "
                      f"{full_us / 1e6:.2f} s",
            "us_per_step_extrapolated": round(full_us, 1), "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
