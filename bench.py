#!/usr/bin/env python3
"""Throughput of attention-score-based KV-cache selection on one MI355X.

Workload: Llama-3.1-8B-shaped prefill compression of all 32 layers, batch 1, L = 32768 prefix tokens, Hq = 32, Hkv = 8, d = 128, bf16,
observation window w = 32, max pool 7, budget k = 2048 per KV head; keys
N(0,1)/sqrt(d) with 1% planted positions in runs of 1-16 tokens (seeded
synthetic inputs, generated on the GPU before timing).

A step is one kvsel_compress per layer (scores -> pool -> top-k -> gather)
for all 32 layers, with every input resident in HBM, the layers processed
one after another on one stream.  The layers' compressions are independent
of one another (each layer is compressed when its prefill ends, while the
next layer's prefill runs), so the same step is also timed with the layers
spread over --overlap-streams streams (layer l on stream l mod S, each with
its own workspace, forked from and joined to the timed stream), where one
layer's small latency-bound kernels overlap another's score passes; that
figure is reported beside the main one.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
METRIC = "prefix tokens scored+compressed/sec (all heads, 1 GPU); % of HBM peak"


def algorithmic_flops(spec):
    """The method's MFMA work: two passes of the logits, 2 H_q w' d flop per
    key each (the recompute in pass 2 included)."""
    return 2 * 2 * spec.Hq * spec.rows * spec.d * sum(spec.seq_lens)


def algorithmic_bytes(spec, kept_rows: int):
    """Bytes the path must move at least once per layer: K read once, Q read,
    the kept K and V rows read and written, and the kept indices written."""
    d = spec.d
    keys = sum(spec.seq_lens)
    k_bytes = keys * spec.Hkv * d * 2
    q_bytes = spec.batch * spec.rows * spec.Hq * d * 2
    gather = kept_rows * d * 2 * 2 * 2
    idx = kept_rows * 4
    return {"K": k_bytes, "Q": q_bytes, "scores_out": keys * spec.Hkv * 4,
            "path": k_bytes + q_bytes + gather + idx}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "kvsel_traffic_llama8b_L32k.json")
# The kernels' code, and the host code that picks their launch shapes.
TRAFFIC_SOURCES = [os.path.join(ROOT, "attention_token_selection_amd", "csrc", f)
                   for f in ("score.hip", "select.hip", "kvsel_device.h", "kvsel_internal.h", "kvsel_api.cpp")]


def source_digest():
    """SHA-256 over the sources the c2 chain's kernels are built from."""
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic():
    """HBM bytes per launch of each kernel of the c2 chain, measured with the
    FETCH_SIZE / WRITE_SIZE counters (record under profiles/), or None once
    the kernels' sources differ from the ones the counters were taken on."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha256") != source_digest():
        return None
    return rec.get("kernels")


def _stats(xs):
    """Median, 10th and 90th percentile (nearest rank) of a list."""
    xs = sorted(xs)
    n = len(xs)

    def q(f):
        return xs[min(n - 1, max(0, int(round(f * (n - 1)))))]

    return {"median": statistics.median(xs), "p10": q(0.1), "p90": q(0.9), "n": n}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def input_digests(torch, cases):
    """SHA-256 of every input buffer (per layer: Q, K, V), over their bytes."""
    out = []
    for c in cases:
        d = {}
        for name in ("Q", "K", "V"):
            t = c[name].contiguous().view(-1).view(torch.uint8).cpu().numpy()
            d[name] = hashlib.sha256(t.tobytes()).hexdigest()
        out.append(d)
    return out


# The c2 chain's kernels, by the start of their names in a kernel trace.
CHAIN_KERNELS = {
    "pass1": "score_kernel<1, 1, false, false>",
    "pass2_tables": "score_kernel<2, 1, false, true>",
    "select_block": "select_block_kernel<true>",
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def summarize_pmc(root, copy_mib):
    """The traffic record from four rocprofv3 --pmc runs under `root`
    (fetch/, write/: the bench; copy_fetch/, copy_write/: the calibration
    copy of copy_mib MiB): per kernel of the c2 chain, the median of
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
    same counter reads for the plain copy."""
    import csv
    import glob

    def read(sub, counter):
        vals = {}
        for f in glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row.get("Kernel_Name", "").replace("(anonymous namespace)::", "")
                    vals.setdefault(name, []).append(float(row["Counter_Value"]))
        return vals

    def pick(vals, prefix):
        xs = [v for n, vs in vals.items() if prefix in n for v in vs]
        return (statistics.median(xs), len(xs)) if xs else (None, 0)

    copy_bytes = copy_mib * 2 ** 20
    cf, _ = pick(read("copy_fetch", "FETCH_SIZE"), COPY_KERNEL)
    cw, _ = pick(read("copy_write", "WRITE_SIZE"), COPY_KERNEL)
    ffac, wfac = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fetch, write = read("fetch", "FETCH_SIZE"), read("write", "WRITE_SIZE")
    kernels = {}
    for key, prefix in CHAIN_KERNELS.items():
        f, nf = pick(fetch, prefix)
        w, nw = pick(write, prefix)
        if f is None or w is None:
            continue
        kernels[key] = {"kernel": prefix, "fetch_kib_median": f, "write_kib_median": w,
                        "fetch_bytes_per_launch": f * 1024 * ffac, "write_bytes_per_launch": w * 1024 * wfac,
                        "bytes_per_launch": f * 1024 * ffac + w * 1024 * wfac, "dispatches": [nf, nw]}
    return {"calibration": {"copy_bytes": copy_bytes, "fetch_kib_counted": cf, "write_kib_counted": cw,
                            "fetch_factor": ffac, "write_factor": wfac},
            "kernels": kernels, "source_sha256": source_digest(),
            "source_files": [os.path.relpath(f, ROOT) for f in TRAFFIC_SOURCES]}


def cpu_baseline(spec, cases, budget_s):
    """The fp64 oracle, untuned, on the host cores (BLAS threads = the cores
    this process may run on): whole c2 layers (all KV heads) until about
    ``budget_s`` seconds of oracle time have been spent; and the c1 workload
    three times on all those cores and three times on one."""
    import oracle.kvsel_oracle as O
    import workloads as W

    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl

        limit = threadpoolctl.threadpool_limits
    except Exception:  # pragma: no cover - informational only
        limit = None

    def run_layers():
        total, tokens, layers = 0.0, 0, 0
        for layer in range(spec.layers):
            c = cases[layer]
            Q = c["Q"].to("cpu").double().numpy()
            K = c["K"].to("cpu").double().numpy()
            V = c["V"].to("cpu").double().numpy()
            t0 = time.perf_counter()
            O.compress(Q, K, V, **W.oracle_kwargs(spec))
            total += time.perf_counter() - t0
            tokens += sum(spec.seq_lens)
            layers += 1
            del Q, K, V
            if total >= budget_s:
                break
        return total, tokens, layers

    def run_c1(threads):
        s1 = W.config(1)
        c = W.make_case(s1)
        Q, K, V = (c[x].double().numpy() for x in "QKV")
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            if limit is not None:
                with limit(limits=threads):
                    O.compress(Q, K, V, **W.oracle_kwargs(s1))
            else:
                O.compress(Q, K, V, **W.oracle_kwargs(s1))
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        return {"tokens_per_s": sum(s1.seq_lens) / med, "seconds_median": med, "runs": 3, "threads": threads}

    if limit is not None:
        with limit(limits=cores):
            total, tokens, layers = run_layers()
    else:
        total, tokens, layers = run_layers()
    return {"value": tokens / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"layers 0-{layers - 1} of {spec.layers} (all {spec.Hkv} KV heads, L={spec.seq_lens[0]}), "
                      f"{total:.1f} s of numpy fp64 oracle time on the host, BLAS threads = {cores}",
            "c1_all_cores": run_c1(cores), "c1_single_core": run_c1(1)}


def _graph_ms(torch, stream, fn, reps):
    """Milliseconds of one replay of the launches `fn` makes, captured into a
    graph: median, p10 and p90 over `reps` replays after a warm-up replay,
    each between its own pair of events on the stream."""
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps + 1):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del g
    return _stats(times[1:])


def time_variants(kv, W, spec, cases, outs, stream, reps):
    """The same 32 layers through the DeferKV variant (one decode-step row,
    exponential row weights with lambda 0.1, 16 sinks and 32 recent kept), the
    same with the guide's mean query per group, TideKV's bounded-memory
    streaming form (8192 keys per step), and KVDrive's warm-up (profile over
    all layers, then the three-tier ranking with 2048 fast and 8192 middle
    slots)."""
    import torch

    dev = cases[0]["K"].device
    L = spec.seq_lens[0]
    g = torch.Generator(device=dev)
    g.manual_seed(20261203)
    # the first decode step's query: one more observation row per layer
    Qd = []
    for c in cases:
        row = torch.randn(spec.batch, 1, spec.Hq, spec.d, generator=g, device=dev) * (spec.d ** 0.5)
        Qd.append(torch.cat([c["Q"], row.to(torch.bfloat16)], dim=1).contiguous())
    res = {}
    base = W.problem_kwargs(spec)
    for name, extra in (("deferkv_exp0.1_sink16_recent32", dict(gqa="sum")),
                        ("deferkv_exp0.1_sink16_recent32_mean_query", dict(gqa="mean"))):
        kw = dict(base, has_decode=True, weighting="exp", lam=0.1, sink=16, recent=32, **extra)
        pv = kv.Problem(**kw)
        wsb, _ = kv.kvsel_plan(pv)
        wsv = torch.empty(wsb, dtype=torch.uint8, device=dev)
        calls = [kv.bind_compress(pv, q, c["K"], c["V"], o["idx"], o["K_out"], o["V_out"], None, wsv, stream)
                 for q, c, o in zip(Qd, cases, outs)]

        def run():
            for call in calls:
                call()

        st = _graph_ms(torch, stream, run, reps)
        ms = st["median"]
        res[name] = {"ms_per_step": ms, "ms_p10": st["p10"], "ms_p90": st["p90"],
                     "tokens_per_s": L * spec.layers * spec.batch / (ms * 1e-3),
                     "what": "kvsel_compress per layer, 32 layers, w'=33 (decode row), k=2048"}
        del wsv
    # TideKV's bounded-memory streaming form: the same selection in steps of
    # 8192 keys, with a workspace that does not grow with the prefix
    for C in (8192, 16384):
        ps = kv.Problem(**dict(base, stream_keys=C))
        wsb, _ = kv.kvsel_plan(ps)
        wss = torch.empty(wsb, dtype=torch.uint8, device=dev)
        calls = [kv.bind_compress(ps, c["Q"], c["K"], c["V"], o["idx"], o["K_out"], o["V_out"], None, wss, stream)
                 for c, o in zip(cases, outs)]

        def run_s():
            for call in calls:
                call()

        st = _graph_ms(torch, stream, run_s, reps)
        ms = st["median"]
        whole = kv.kvsel_plan(kv.Problem(**base))[0]
        res[f"tidekv_streaming_{C}"] = {
            "ms_per_step": ms, "ms_p10": st["p10"], "ms_p90": st["p90"],
            "tokens_per_s": L * spec.layers * spec.batch / (ms * 1e-3),
            "workspace_MiB": wsb / 2 ** 20, "whole_prefix_workspace_MiB": whole / 2 ** 20,
            "what": f"kvsel_compress with stream_keys={C}, 32 layers, k=2048"}
        del wss
    pw = kv.Problem(**dict(base, pool="none"))
    wsb, _ = kv.kvsel_plan(pw)
    wsw = torch.empty(wsb, dtype=torch.uint8, device=dev)
    prof = torch.empty(sum(spec.seq_lens), dtype=torch.float32, device=dev)
    tier = torch.empty(sum(spec.seq_lens), dtype=torch.int8, device=dev)

    def warm():
        for l, c in enumerate(cases):
            kv.kvsel_profile_layer(pw, c["Q"], c["K"], prof, wsw, accumulate=l > 0, stream=stream)
        kv.kvsel_tier_rank(pw, prof, 2048, 8192, tier, wsw, stream=stream)

    st = _graph_ms(torch, stream, warm, reps)
    ms = st["median"]
    res["kvdrive_warmup_32layers_tiers_2048_8192"] = {
        "ms_per_step": ms, "ms_p10": st["p10"], "ms_p90": st["p90"],
        "tokens_per_s": L * spec.layers * spec.batch / (ms * 1e-3),
        "what": "kvsel_profile_layer for 32 layers, then kvsel_tier_rank"}
    return res


def time_workloads(kv, W, stream, reps, skip):
    """Every workload of the measurement plan other than the headline one
    (index `skip`), each as one kvsel_compress call replayed from a graph:
    milliseconds per call, prefix tokens per second, and the path's
    algorithmic bytes (K once, Q, kept K/V read and written, indices) per
    second against HBM peak.  Reported beside the headline figure."""
    import torch

    dev = torch.device("cuda:0")
    res = {}
    for i in range(1, 6):
        if i == skip:
            continue
        spec = W.config(i)
        case = W.make_case(spec, device=dev)
        p = kv.Problem(**W.problem_kwargs(spec))
        out = kv.alloc_outputs(p, dev, pooled=False)
        call = kv.bind_compress(p, case["Q"], case["K"], case["V"], out["idx"], out["K_out"], out["V_out"],
                                None, out["ws"], stream)
        st = _graph_ms(torch, stream, call, reps)
        ms = st["median"]
        kept = kv.kvsel_plan(p)[1][-1]
        ab = algorithmic_bytes(spec, kept)
        tokens = sum(spec.seq_lens)
        hbm = ab["path"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
        mfma = algorithmic_flops(spec) / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS
        # the binding roof is the slower of the two at full rate
        t_hbm = ab["path"] / (HBM_PEAK_GBS * 1e9)
        t_mfma = algorithmic_flops(spec) / (MFMA_PEAK_TFLOPS * 1e12)
        res[spec.name] = {
            "ms_per_call": ms, "ms_p10": st["p10"], "ms_p90": st["p90"], "tokens_per_s": tokens / (ms * 1e-3),
            "path_GBps": ab["path"] / (ms * 1e-3) / 1e9, "hbm_frac_path": hbm, "mfma_frac": mfma,
            "binding_roof": "mfma" if t_mfma > t_hbm else "hbm", "binding_frac": max(t_hbm, t_mfma) / (ms * 1e-3),
            "tokens": tokens, "kept_rows": kept,
            "resident_in_infinity_cache": ab["K"] * 2 < 256 * 2 ** 20,
        }
        del case, out, call
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--graph", type=int, default=1, help="replay each step from a captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time the CPU baseline runs for, in whole layers (0: skip)")
    ap.add_argument("--stage-reps", type=int, default=9,
                    help="graph replays per stage / variant / workload figure (median, p10, p90 reported)")
    ap.add_argument("--streams", type=int, default=1,
                    help="spread the layers' independent compressions over this many streams (layer l on "
                         "stream l mod S, each with its own workspace), forked from and joined to the timed "
                         "stream; 1 (default) processes the layers one after another")
    ap.add_argument("--overlap-streams", type=int, default=4,
                    help="also time the same step with the layers spread over this many streams, reported "
                         "beside the main figure (0: skip)")
    ap.add_argument("--variants", type=int, default=1,
                    help="also time the DeferKV and KVDrive warm-up variants on the same layers (0: skip)")
    ap.add_argument("--workloads", type=int, default=1,
                    help="also time one kvsel_compress call of each other workload of the measurement plan "
                         "(reported beside the main figure; 0: skip)")
    ap.add_argument("--digests", type=int, default=1,
                    help="record a SHA-256 of every input buffer (per layer: Q, K, V) in the line")
    ap.add_argument("--variants-only", type=int, default=0,
                    help="only time the variants and print them (for a kernel trace of the variants alone)")
    ap.add_argument("--summarize-pmc", default="", metavar="DIR",
                    help="(no GPU) print the traffic record from the four rocprofv3 --pmc runs under DIR "
                         "(fetch/, write/, copy_fetch/, copy_write/) and exit")
    ap.add_argument("--summarize-copy-mib", type=int, default=256)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's plain device copy of MIB MiB (5 times) and exit: the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc, args.summarize_copy_mib), indent=1))
        return
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              "(each GPU would take whole (sequence, KV head) segments independently).", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_MiB": args.copy_calibration, "copies": 5}), flush=True)
        return

    import attention_token_selection_amd as kv
    import workloads as W

    spec = W.config(2)
    L = spec.seq_lens[0]
    print(f"[bench] generating {spec.layers} layers of {spec.name} on {dev}", file=sys.stderr, flush=True)
    cases = [W.make_case(spec, layer=l, device=dev) for l in range(spec.layers)]
    p = kv.Problem(**W.problem_kwargs(spec))
    ws_bytes, offs = kv.kvsel_plan(p)
    kept = offs[-1]
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = [kv.alloc_outputs(p, dev, pooled=False) for _ in range(spec.layers)]
    for o in outs:
        o["ws"] = ws  # one workspace: the layers run one after another on one stream

    stream = torch.cuda.Stream(device=dev)
    if args.variants_only:
        print(json.dumps({"variants": time_variants(kv, W, spec, cases, outs, stream, args.stage_reps)}), flush=True)
        return
    def make_step(n_streams):
        """The 32 layers' kvsel_compress calls, on one stream or spread over
        n_streams forked from (and joined back to) the timed stream."""
        side = [stream] if n_streams == 1 else [torch.cuda.Stream(device=dev) for _ in range(n_streams)]
        side_ws = [ws] + [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(n_streams - 1)]
        calls = [kv.bind_compress(p, c["Q"], c["K"], c["V"], o["idx"], o["K_out"], o["V_out"], None,
                                  side_ws[l % n_streams], side[l % n_streams])
                 for l, (c, o) in enumerate(zip(cases, outs))]

        def step():
            if n_streams > 1:
                for st in side:
                    st.wait_stream(stream)
            for call in calls:
                call()
            if n_streams > 1:
                for st in side:
                    stream.wait_stream(st)

        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        if not args.graph:
            return step, (side, side_ws, calls)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()
        return graph.replay, (side, side_ws, calls, graph)

    n_streams = max(1, args.streams)
    run, keep_alive = make_step(n_streams)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run()
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for a, b in step_ev:
            a.record(stream)
            run()
            b.record(stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall = t1 - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    elapsed = max(wall, gpu_s)
    tokens_per_step = L * spec.layers * spec.batch
    value = tokens_per_step * args.steps / elapsed
    ms_per_step = elapsed / args.steps * 1e3
    step_ms = _stats([a.elapsed_time(b) for a, b in step_ev])

    overlap = None
    if args.overlap_streams > 1 and n_streams == 1:
        run_o, keep_o = make_step(args.overlap_streams)
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                run_o()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(args.steps):
                run_o()
            b.record(stream)
        torch.cuda.synchronize()
        ms_o = a.elapsed_time(b) / args.steps
        overlap = {"streams": args.overlap_streams, "ms_per_step": ms_o,
                   "tokens_per_s": tokens_per_step / (ms_o * 1e-3),
                   "what": "the same 32 layers with their independent compressions spread over streams"}
        del run_o, keep_o

    ab = algorithmic_bytes(spec, kept)
    path_gbs = ab["path"] * spec.layers * args.steps / elapsed / 1e9
    path_gbs_median = ab["path"] * spec.layers / (step_ms["median"] * 1e-3) / 1e9

    # Per-stage timing with HIP events on the library's stream: each stage is
    # launched for all layers back to back, captured into a graph (so that
    # the host's submission speed does not show), and replayed stage_reps
    # times, each replay between its own pair of events.
    #   pass1     kvsel_row_stats: score pass 1 alone
    #   pass1+2t  kvsel_compress with every budget 0: pass 1, pass 2 with the
    #             pool and selection tables, and a selection launch whose
    #             workgroups all leave at once (nothing to keep)
    #   compress  kvsel_compress: the whole step
    #   score, pool_topk, gather: the step's other entry points
    scores = torch.empty(sum(spec.seq_lens) * spec.Hkv, dtype=torch.float32, device=dev)
    p0 = kv.Problem(**dict(W.problem_kwargs(spec), k=0))
    ws0 = torch.empty(kv.kvsel_plan(p0)[0], dtype=torch.uint8, device=dev)
    stage = {}
    for name in ("pass1", "pass1+2t", "compress", "score", "pool_topk", "gather"):
        def launch_all():
            for c, o in zip(cases, outs):
                if name == "pass1":
                    kv.kvsel_row_stats(p, c["Q"], c["K"], ws, stream)
                elif name == "pass1+2t":
                    kv.kvsel_compress(p0, c["Q"], c["K"], c["V"], None, None, None, None, ws0, stream)
                elif name == "compress":
                    kv.kvsel_compress(p, c["Q"], c["K"], c["V"], o["idx"], o["K_out"], o["V_out"], None, ws, stream)
                elif name == "score":
                    kv.kvsel_score(p, c["Q"], c["K"], scores, ws, stream)
                elif name == "pool_topk":
                    kv.kvsel_pool_topk(p, scores, None, o["idx"], ws, stream)
                else:
                    kv.kvsel_gather(p, o["idx"], c["K"], c["V"], o["K_out"], o["V_out"], stream)

        st = _graph_ms(torch, stream, launch_all, args.stage_reps)
        stage[name] = {k: (v * 1e3 / len(cases) if k != "n" else v) for k, v in st.items()}  # us per layer
    del ws0
    stage_us = {k: v["median"] for k, v in stage.items()}
    # The chain's three kernels' launch times: pass 1 alone, pass 2 with
    # tables as the difference (its empty selection launch stays in it), and
    # the selection as the rest of the whole step.
    t_pass1 = stage_us["pass1"]
    t_pass2 = stage_us["pass1+2t"] - stage_us["pass1"]
    t_select = stage_us["compress"] - stage_us["pass1+2t"]
    traffic = counted_traffic() or {}
    kernels = {
        "pass1": {
            "kernel": "score pass 1: logits + row statistics (score_kernel<1>)",
            "us_per_launch": t_pass1,
            "algorithmic_bytes": ab["K"] + ab["Q"],
            "what_bytes": "K read once + Q",
            "traffic": (traffic.get("pass1") or {}).get("bytes_per_launch"),
        },
        "pass2_tables": {
            "kernel": "score pass 2 with pool and selection tables (score_kernel<2, .., TAB>)",
            "us_per_launch": t_pass2,
            # K again (the method's recompute) and Q; pooled scores and the
            # tables of every 256 positions (2048 u16 prefix + 256 u32 keys)
            "algorithmic_bytes": ab["K"] + ab["Q"] + ab["scores_out"] + sum(spec.seq_lens) * spec.Hkv * 20,
            "what_bytes": "K + Q read; pooled scores (4 B) and selection tables (20 B) per position written",
            "traffic": (traffic.get("pass2_tables") or {}).get("bytes_per_launch"),
        },
        "select_block": {
            "kernel": "selection from the tables, ordered compaction and K/V gather (select_block_kernel<true>)",
            "us_per_launch": t_select,
            "algorithmic_bytes": ab["path"] - ab["K"] - ab["Q"],
            "what_bytes": "kept K and V rows read and written, kept indices written",
            "traffic": (traffic.get("select_block") or {}).get("bytes_per_launch"),
        },
    }
    for k in kernels.values():
        k["achieved_GBps"] = k["algorithmic_bytes"] / (k["us_per_launch"] * 1e-6) / 1e9
        k["frac"] = k["achieved_GBps"] / HBM_PEAK_GBS
    dom = max(kernels, key=lambda n: kernels[n]["us_per_launch"])

    variants = time_variants(kv, W, spec, cases, outs, stream, args.stage_reps) if args.variants else None
    workloads = time_workloads(kv, W, stream, args.stage_reps, skip=2) if args.workloads else None

    cpu = None
    if args.cpu_seconds > 0:
        print(f"[bench] cpu oracle baseline, about {args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        cpu = cpu_baseline(spec, cases, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {
            "workload": "llama3.1-8b-shaped prefill KV selection: 32 layers processed one after another, "
                        "batch 1, L=32768, Hq=32, Hkv=8, d=128, w=32, max pool 7, k=2048 per KV head",
            "layers": spec.layers, "batch": spec.batch, "seq_len": L, "graph": bool(args.graph),
            "streams": n_streams,
        },
        "step_ms": step_ms,
        "hbm_frac_path": path_gbs / HBM_PEAK_GBS,
        "hbm_frac_path_median_step": path_gbs_median / HBM_PEAK_GBS,
        "path_GBps": path_gbs,
        "stage_us": stage_us,
        "stage_us_p10_p90": {k: [v["p10"], v["p90"]] for k, v in stage.items()},
        "roofline": {
            "kernel": kernels[dom]["kernel"],
            "bound": "hbm",
            "achieved": kernels[dom]["achieved_GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": kernels[dom]["frac"],
            "traffic": kernels[dom]["traffic"],
            "path_frac": path_gbs / HBM_PEAK_GBS,
            "kernels": kernels,
        },
        "input_sha256": input_digests(torch, cases) if args.digests else None,
        "cpu_baseline": cpu,
        "variants": variants,
        "other_workloads": workloads,
        "overlapped_layers": overlap,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
