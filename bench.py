#!/usr/bin/env python3
"""Benchmark: paged split-KV GQA decode attention on one MI355X.

One step = pa_decode_run + pa_decode_combine (split-KV decode kernel + combine
kernel) over the whole batch, on one stream, with every input resident in HBM
(--fused-combine merges inside the decode kernel instead).  The plan is built once
before timing (it is reusable while lengths are unchanged) and timed separately.
Headline workload (--config, default 1): GQA decode at a Llama-70B-like shape (B=32,
Hq=64, Hkv=8, D=128, bf16 KV, 64-token pages, 4096 tokens each, balanced plan).

Prints ONE JSON line.  `value` is the headline workload's achieved algorithmic KV
bandwidth (GB/s) of a whole step; `roofline` is for its dominant kernel (the decode
kernel), timed with HIP events on the launch stream over a graph of back-to-back
launches (its device time; eager launches of a small kernel time the host's launch
rate instead); `cpu_baseline` times the fp64 CPU oracle on a bounded sample of the
same workload.  `workloads` holds the same measurements, lighter, for every named
workload (tiny, Llama-70B-like, HD64 at B=1 and B=8, ragged FP8, MLA).  A workload
whose KV pool fits in the 256 MB last-level cache is also timed cold (each step reads
the next of enough pool copies to exceed 512 MB), and its roofline figure is the cold
one.
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
# the workloads of the `workloads` record: (index, batch)
ALL_WORKLOADS = ((0, None), (1, None), (2, 1), (2, 8), (3, None), (4, None))


def counter_traffic(workload, batch):
    """Calibrated HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings, and where they come from; (None, None)
    when the kernel source has changed since they were taken (or none were taken)."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)
        w = rec["workloads"]["%s, B=%d" % (workload, batch)]
        with open(os.path.join(ROOT, w["source"]), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if sha != w["source_sha256"]:
            return None, None
        nbytes = int(round(w["fetch_kib"] * 1024 * rec["fetch_factor"]
                           + w["write_kib"] * 1024 * rec["write_factor"]))
        return nbytes, ("profiles/traffic.json: rocprofv3 FETCH_SIZE / WRITE_SIZE of %s at "
                        "%s sha256 %s (not counted in this run)" % (w["kernel"], w["source"], sha[:16]))
    except (OSError, KeyError, ValueError):
        return None, None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="headline workload index (default 1)")
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
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only the headline workload (no `workloads` record)")
    ap.add_argument("--cold-copies", type=int, default=-1,
                    help="also time with each step reading the next of N copies of the KV pool "
                         "(so that the pool is not cache-resident); -1: automatic (enough copies "
                         "to exceed 512 MB when one pool fits in the 256 MB last-level cache), 0: off")
    ap.add_argument("--fused-combine", action="store_true",
                    help="merge chunks inside the decode kernel (last workgroup per request) "
                         "instead of the combine kernel")
    return ap.parse_args()


class Workload:
    """One workload's device tensors, runner and step."""

    def __init__(self, case, fused=False, q_len=1):
        import numpy as np
        import torch

        from mqa_split_kv_amd import binding as pb

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).cuda()

        self.case = case
        self.q = dev(case["q"])
        self.kp = dev(case["k_pool"])
        self.vp = dev(case["v_pool"]) if case.get("v_pool") is not None else None
        self.ks = dev(case["k_scale"]) if case.get("k_scale") is not None else None
        self.vs = dev(case["v_scale"]) if case.get("v_scale") is not None else None
        self.bt, self.sl = dev(case["block_table"]), dev(case["seq_lens"])
        self.idx = dev(case["indices"]) if case.get("topk") else None
        B, Hq, Dv = case["B"], case["Hkv"] * case["G"], case["Dv"]
        self.out = torch.empty((B, q_len, Hq, Dv), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device="cuda")
        self.desc = pb.desc_from_case(case, fused=fused)
        self.runner = pb.PagedDecode(self.desc)
        self.stream = torch.cuda.current_stream()
        self.runner.plan(self.sl)

    def run(self, pools=None):
        kp, vp, ks, vs = pools if pools is not None else (self.kp, self.vp, self.ks, self.vs)
        self.runner.run(self.q, kp, vp, self.bt, self.sl, self.out, self.lse, k_scale=ks, v_scale=vs,
                        indices=self.idx)

    def step(self, pools=None):
        self.run(pools)
        self.runner.combine(self.out, self.lse)

    def pool_bytes(self):
        return sum(t.numel() * t.element_size() for t in (self.kp, self.vp, self.ks, self.vs) if t is not None)


def events_us(stream, fn, n):
    """Device µs per call of fn, over n calls bracketed by HIP events on `stream`."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / n


def graph_us(fn, per_graph, reps):
    """Device µs per call of fn from a captured graph of `per_graph` calls replayed `reps`
    times (the per-replay launch cost is amortised)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (reps * per_graph), g


def time_workload(w, steps, warmup, graph=True, protocol=False, cold_copies=-1):
    """Step (eager), decode kernel (eager and from a graph), graph step, optional grouped
    protocol and cold timing, in µs."""
    import numpy as np
    import torch

    for _ in range(warmup):
        w.step()
    torch.cuda.synchronize()
    r = {"us_per_step": events_us(w.stream, w.step, steps)}
    r["decode_kernel_us"] = events_us(w.stream, w.run, max(steps, 50))
    w.runner.combine(w.out, w.lse)
    torch.cuda.synchronize()
    r["graph_us_per_step"] = r["decode_kernel_graph_us"] = None
    g = None
    if graph:
        per_graph = 20
        reps = max(1, steps // per_graph)
        r["graph_us_per_step"], g = graph_us(lambda i: w.step(), per_graph, reps)
        r["decode_kernel_graph_us"], _ = graph_us(lambda i: w.run(), per_graph, reps)
        w.runner.combine(w.out, w.lse)
        torch.cuda.synchronize()
    r["timing_protocol"] = None
    if protocol:
        # the MetaX page's protocol: 10 groups of 100 calls after the warm-ups, median of
        # the group means, eager and from graphs (of 20 calls each)
        groups, calls = 10, 100

        def median_of_groups(one_group):
            return round(float(np.median([events_us(w.stream, one_group, 1) / calls for _ in range(groups)])), 2)

        def eager_group():
            for _ in range(calls):
                w.step()
        proto = {"groups": groups, "calls_per_group": calls,
                 "eager_us_median": median_of_groups(eager_group), "graph_us_median": None}
        if g is not None:
            def graph_group():
                for _ in range(calls // 20):
                    g.replay()
            proto["graph_us_median"] = median_of_groups(graph_group)
        r["timing_protocol"] = proto
    del g
    r["cold"] = None
    pool = w.pool_bytes()
    n = cold_copies
    if n < 0:
        n = min(-(-(512 << 20) // pool) + 1, 1024) if pool < (256 << 20) else 0
    if n > 0:
        r["cold"] = cold_timing(w, n, steps, graph)
    for k in ("us_per_step", "decode_kernel_us", "graph_us_per_step", "decode_kernel_graph_us"):
        if r[k] is not None:
            r[k] = round(r[k], 2)
    return r


def cold_timing(w, ncopies, steps, graph):
    """The step, the decode kernel and a graph of steps, each step reading the next of
    `ncopies` copies of the KV pool (and scales): with more bytes than the last-level
    cache holds, every step's KV comes from HBM."""
    import torch

    copies = [tuple(None if t is None else t.clone() for t in (w.kp, w.vp, w.ks, w.vs)) for _ in range(ncopies)]
    torch.cuda.synchronize()
    n = max(steps, 2 * ncopies)
    k = [0]

    def step():
        w.step(copies[k[0] % ncopies])
        k[0] += 1

    def run():
        w.run(copies[k[0] % ncopies])
        k[0] += 1

    for _ in range(ncopies):
        step()
    res = {"copies": ncopies, "bytes_rotated": w.pool_bytes() * ncopies,
           "us_per_step": round(events_us(w.stream, step, n), 2),
           "decode_kernel_us": round(events_us(w.stream, run, n), 2),
           "graph_us_per_step": None, "decode_kernel_graph_us": None}
    w.runner.combine(w.out, w.lse)
    if graph:
        reps = max(2, n // ncopies)
        res["graph_us_per_step"] = round(graph_us(lambda i: w.step(copies[i]), ncopies, reps)[0], 2)
        res["decode_kernel_graph_us"] = round(graph_us(lambda i: w.run(copies[i]), ncopies, reps)[0], 2)
        w.runner.combine(w.out, w.lse)
    torch.cuda.synchronize()
    del copies
    torch.cuda.empty_cache()
    return res


def roofline(case, t, q_len=1, topk=0):
    """Roofline of the dominant kernel (the decode kernel) from its device time: a cold
    figure when the workload was timed cold, else the graph-timed one (eager when no
    graph was timed)."""
    from mqa_split_kv_amd import synth

    kv = synth.kv_bytes(case)
    cold = t.get("cold")
    if cold is not None:
        us = cold["decode_kernel_graph_us"] or cold["decode_kernel_us"]
        timing = "cold (%d rotating pool copies)" % cold["copies"]
    else:
        us = t["decode_kernel_graph_us"] or t["decode_kernel_us"]
        timing = "warm"
    timing += ", graph of launches" if t["decode_kernel_graph_us"] is not None else ", eager launches"
    if case["kv_format"] == synth.KV_MLA656:
        # MLA: 128 heads share each token, so the contraction is MFMA-bound
        tokens = kv / synth.MLA_TOKEN_BYTES            # attended keys (listed ones if sparse)
        tflops = MLA_FLOP_PER_TOKEN * q_len * tokens / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "kernel": "pa_mla_kernel", "kernel_us": us, "timing": timing,
                "algorithmic_flop": int(MLA_FLOP_PER_TOKEN * q_len * tokens)}
    gbs = kv / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": "pa_decode_kernel<%d,%s>" % (case["D"], "bf16" if case["kv_format"] == 0 else "fp8"),
            "kernel_us": us, "timing": timing, "algorithmic_bytes": kv}


def workload_record(case, t, index, q_len=1, topk=0):
    """The per-workload summary of the `workloads` record."""
    import numpy as np

    from mqa_split_kv_amd import synth

    kv = synth.kv_bytes(case)
    rec = {"index": index, "workload": case["name"], "B": case["B"], "Hq": case["Hkv"] * case["G"],
           "Hkv": case["Hkv"], "D": case["D"], "Dv": case["Dv"], "page_size": case["page_size"],
           "seq_len_total": int(np.sum(case["seq_lens"])), "kv_format": fmt_name(case),
           "num_splits": "balanced plan" if case["num_splits"] == 0 else case["num_splits"],
           "kv_bytes_per_step": kv,
           "us_per_step": t["us_per_step"], "graph_us_per_step": t["graph_us_per_step"],
           "decode_kernel_us": t["decode_kernel_us"], "decode_kernel_graph_us": t["decode_kernel_graph_us"],
           "kv_gbs_step": round(kv / (t["us_per_step"] * 1e-6) / 1e9, 1),
           "roofline": roofline(case, t, q_len, topk), "cold": t["cold"]}
    if t["graph_us_per_step"]:
        rec["kv_gbs_graph_step"] = round(kv / (t["graph_us_per_step"] * 1e-6) / 1e9, 1)
    ref = PAGES_GRAPH_US.get((index, case["B"]))
    if ref is not None and t["graph_us_per_step"]:
        rec["pages_graph_us_per_call"] = ref
        rec["pages_context"] = ("MetaX C500 25 % slice, same step and timing protocol (MetaX PR page, "
                                "performance table): another machine, context only")
    traffic, source = counter_traffic(case["name"], case["B"]) if q_len == 1 and not topk else (None, None)
    rec["roofline"]["traffic"] = traffic
    rec["roofline"]["traffic_source"] = source
    return rec


def fmt_name(case):
    return {0: "bf16", 1: "fp8e4m3-kv/bf16", 2: "mla656-fp8/bf16"}[case["kv_format"]]


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
    print(f"[bench] generated workload {args.config} ({case['name']}) in {time.time() - t_gen:.1f}s",
          file=sys.stderr, flush=True)
    w = Workload(case, fused=args.fused_combine, q_len=args.q_len)

    # plan (once; timed separately: eager launches, and from a graph for its device time)
    plan_us = events_us(w.stream, lambda: w.runner.plan(w.sl), 10)
    plan_graph_us = None if args.no_graph else round(graph_us(lambda i: w.runner.plan(w.sl), 20, 5)[0], 2)
    w.step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps bracketed by synchronisation
    for _ in range(args.warmup):
        w.step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    step_us = events_us(w.stream, w.step, args.steps)
    wall_s = time.perf_counter() - w0
    t = time_workload(w, args.steps, 0, graph=not args.no_graph, protocol=not args.no_protocol,
                      cold_copies=args.cold_copies)
    t["us_per_step"] = round(step_us, 2)

    kv_bytes = synth.kv_bytes(case)
    io = synth.io_bytes(case)
    gbs = kv_bytes / (step_us * 1e-6) / 1e9
    roof = roofline(case, t, args.q_len, args.topk)
    traffic, source = counter_traffic(case["name"], case["B"]) if args.q_len == 1 and not args.topk else (None, None)
    roof["traffic"] = traffic
    roof["traffic_source"] = source

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

    headline = workload_record(case, t, args.config, args.q_len, args.topk)
    del w
    torch.cuda.empty_cache()

    # every named workload, with a lighter protocol (the headline's record is reused)
    workloads = None
    if not args.no_workloads and args.q_len == 1 and not args.topk and not args.fused_combine:
        workloads = []
        for index, B in ALL_WORKLOADS:
            if index == args.config and (index != 2 or B == case["B"]):
                workloads.append(headline)
                continue
            t0 = time.time()
            c = synth.config_case(index, B=B)
            if index == 0:
                c["num_splits"] = 2                 # the tiny workload's split setting with a combine
            print(f"[bench] workload {index} ({c['name']}, B={c['B']}) generated in {time.time() - t0:.1f}s",
                  file=sys.stderr, flush=True)
            wl = Workload(c)
            tw = time_workload(wl, 50, 5, graph=not args.no_graph, protocol=(index == 2 and not args.no_protocol))
            workloads.append(workload_record(c, tw, index))
            if tw["timing_protocol"]:
                workloads[-1]["timing_protocol"] = tw["timing_protocol"]
            del wl, c
            torch.cuda.empty_cache()
            print(f"[bench] workload {index} timed", file=sys.stderr, flush=True)

    cfg = {"workload": case["name"], "B": case["B"], "Hq": case["Hkv"] * case["G"], "Hkv": case["Hkv"],
           "D": case["D"], "Dv": case["Dv"], "page_size": case["page_size"],
           "seq_len_total": int(np.sum(case["seq_lens"])), "kv_format": fmt_name(case),
           "q_len": args.q_len, "topk": args.topk or None,
           "num_splits": "balanced plan" if case["num_splits"] == 0 else case["num_splits"],
           "num_parts": pb.pa_decode_num_parts(pb.desc_from_case(case)),
           "combine": "fused in the decode kernel" if args.fused_combine else "combine kernel",
           "parallelism": "single GPU"}
    # vs_baseline: only where the pages give a number for this very workload (same step, same
    # timing protocol): their graph µs per call over this run's graph median
    vs_baseline, vs_basis = None, None
    ref_us = PAGES_GRAPH_US.get((args.config, case["B"]))
    proto = t["timing_protocol"]
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
        "ms_per_step": round(step_us / 1000.0, 5),
        "us_per_step": round(step_us, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs_baseline,
        "vs_baseline_basis": vs_basis,
        "dtype": "bf16" if case["kv_format"] == 0 else fmt_name(case),
        "data": "synthetic (seeded N(0,1), random page permutation)",
        "config": cfg,
        "kv_bytes_per_step": kv_bytes,
        "io_bytes_per_step": io,
        "plan_us": round(plan_us, 2),
        "plan_graph_us": plan_graph_us,
        "decode_kernel_us": t["decode_kernel_us"],
        "decode_kernel_graph_us": t["decode_kernel_graph_us"],
        "graph_us_per_step": t["graph_us_per_step"],
        "wall_s_timed": round(wall_s, 4),
        "roofline": roof,
        "cold": None if t["cold"] is None else dict(
            t["cold"], kv_gbs_step=round(kv_bytes / (t["cold"]["us_per_step"] * 1e-6) / 1e9, 1),
            pct_of_hbm_peak_step=round(100.0 * kv_bytes / (t["cold"]["us_per_step"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)),
        "timing_protocol": proto,
        "read_ceiling_gbs": ceiling,
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(rec), flush=True)


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
