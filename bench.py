"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (router, top-k, grouping, expert FFN on
MXFP4 weights, combine) over one batch of synthetic tokens already resident
in HBM.  The default workload is single-token greedy decode on the
896-expert / top-16 layer (d_model 7168, d_ff 2048), a fresh seeded token per
step (1000 distinct tokens, cycled).

Prints one JSON line: throughput in tokens/s; the roofline of the dominant
kernel (its algorithmic bytes -- the active experts' weights it streams, the
activations it reads, the outputs it writes -- over its average time, taken
from HIP events attached to each kernel dispatch of the expert-FFN stage on
the launch stream), with every kernel of the stage and the whole stage
(timed by events around k3moe_ffn) beside it; and the fp64 oracle timed on
the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
# the kernel sources whose counters profiles/traffic.json records
TRAFFIC_SOURCES = ["mxfp4_routed_expert_softmax_amd/csrc/" + f for f in
                   ("gemv.hip", "mx.hip", "slices.hip", "route.hip", "api.hip", "device_common.h", "kernels.h",
                    "slices.h", "topk.h")]
FFN_KERNELS = ("gateup_", "down_", "combine_", "quantize_rows", "zero_kernel", "active_list")
MXFP4_PEAK_TFLOPS = 10100.0  # dense MXFP4 matrix peak
EV_EVERY_DECODE = 10  # one-token steps per event-marked step (others: every step)
MIN_EV_SAMPLES = 10   # event-marked steps per measurement, whatever --steps is
PREFILL_WORKLOAD = "k3_prefill_t4096"  # timed after the headline workload, same run


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="k3_decode_t1")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of host time for the oracle baseline (0 disables it)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step from a captured HIP graph instead of eager launches")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="also time steps with a read of this many MiB between them (caches cold; "
                         "informational, reported under 'flushed')")
    ap.add_argument("--prefill-steps", type=int, default=10,
                    help="timed steps of the 4096-token MXFP4 prefill reported under 'prefill' "
                         "(0 disables it; only with the headline decode workload)")
    ap.add_argument("--cache-slots", type=int, default=256,
                    help="after the headline decode run, the same decode through the HBM expert cache "
                         "(k3moe_forward_cached) with this many expert slots, every expert in pinned host "
                         "memory; 0 skips it")
    ap.add_argument("--cache-steps", type=int, default=200, help="timed steps of the cached decode")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, copy this many MiB three times with the runtime's copy and three "
                         "times with an elementwise kernel (reference kernels for hardware byte counters; "
                         "not part of the step)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer is measured on one GPU: --gpus must be 1 (sharding across GPUs is described, not built)"}))
        sys.exit(2)
    import torch
    import synthdata
    import mxfp4_routed_expert_softmax_amd as k3

    wl = synthdata.WORKLOADS[args.workload]
    sh, T = wl.shape, wl.T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {wl.name}: T={T} E={sh.E} k={sh.k} d={sh.d} f={sh.f} act={wl.act_mode}")

    t0 = time.time()
    experts = synthdata.upload_experts(sh, dev)
    wr = torch.from_numpy(synthdata.router_weight(sh)).to(dev)
    torch.cuda.synchronize()
    log(f"layer resident in {time.time() - t0:.1f}s")

    m = measure(k3, synthdata, torch, dev, wl, experts, wr, args.steps, args.warmup, args.graph)
    fw, xs, nbatch, stream = m["fw"], m["xs"], m["nbatch"], m["stream"]
    ms_per_step, tokens_per_s, roofline = m["ms_per_step"], m["tokens_per_s"], m["roofline"]
    n_active, bias_mode, graph = m["n_active"], m["bias_mode"], m["graph"]

    prefill = None
    if args.prefill_steps > 0 and wl.name == "k3_decode_t1" and not args.graph:
        pw = synthdata.WORKLOADS[PREFILL_WORKLOAD]
        log(f"prefill block: {pw.name}")
        pm = measure(k3, synthdata, torch, dev, pw, experts, wr, args.prefill_steps, 3, False)
        prefill = {"workload": pw.name, "T": pw.T, "activations": pw.act_mode, "steps": args.prefill_steps,
                   "warmup": 3, "ms_per_step": round(pm["ms_per_step"], 5),
                   "tokens_per_s": round(pm["tokens_per_s"], 1), "roofline": pm["roofline"],
                   "active_experts_last_step": pm["n_active"]}
        del pm

    cache = None
    if args.cache_slots > 0 and wl.name == "k3_decode_t1" and not args.graph:
        log(f"cache block: {args.cache_slots} slots")
        cache = measure_cache(k3, synthdata, torch, wl, experts, wr, xs, args.cache_slots, args.cache_steps)

    flushed = None
    if args.flush_mib > 0:
        # each step timed alone by events on this stream, a read of a large
        # buffer (untimed) before it, so that no weight is left in the caches
        buf = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        sink = torch.zeros(1, dtype=torch.float32, device=dev)
        nfl = min(args.steps, 100)
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nfl)]
        for i in range(nfl):
            sink += buf.sum()
            fw.set_x(xs[i % nbatch])
            fev[i][0].record(stream)
            fw()
            fev[i][1].record(stream)
        torch.cuda.synchronize()
        fms = float(np.mean([a.elapsed_time(b) for a, b in fev]))
        flushed = {"mib": args.flush_mib, "steps": nfl, "ms_per_step": round(fms, 5),
                   "tokens_per_s": round(T / (fms * 1e-3), 1)}
        del buf

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)                 # the runtime's blit kernel
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # an elementwise kernel: one 16-byte load and store per lane step
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(sh, wl, args.cpu_seconds)

    out = {
        "metric": "MoE-layer tokens/s at 1 MI355X (single-token decode, 896 experts, top-16)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "E": sh.E, "k": sh.k, "d_model": sh.d, "d_ff": sh.f,
                   "activations": wl.act_mode, "weights": "MXFP4 (E2M1 codes + E8M0 block-32 scales)",
                   "router_bias": bias_mode, "distinct_batches": nbatch,
                   "launch": "hip graph replay" if graph is not None else "eager, one stream",
                   "active_experts_last_step": n_active},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if prefill is not None:
        out["prefill"] = prefill
    if cache is not None:
        out["cache"] = cache
    if flushed is not None:
        out["flushed"] = flushed
    print(json.dumps(out), flush=True)


def measure(k3, synthdata, torch, dev, wl, experts, wr, steps, warmup, use_graph):
    """Time `steps` steps of workload wl (after `warmup`), inputs resident.
    Every ev_every-th step issues k3moe_route and k3moe_ffn as two calls with
    HIP events on the launch stream around the expert-FFN stage; as many
    other steps (the same steps when every step carries events) have the
    library attach start / end events to each kernel dispatch of the stage;
    the rest issue k3moe_forward.  At least MIN_EV_SAMPLES steps carry
    events."""
    sh, T = wl.shape, wl.T
    bias = torch.from_numpy(synthdata.zipf_bias(sh)).to(dev) if wl.zipf_bias else None
    bias_mode = "logits" if wl.zipf_bias else "none"
    # distinct seeded batches, resident in HBM before timing
    nbatch = 1000 if T == 1 else max(1, min(8, 1000 // T))
    xs = [torch.from_numpy(synthdata.tokens(sh, T, first=i * T)).to(dev) for i in range(nbatch)]
    torch.cuda.synchronize()

    fw = k3.Forward(xs[0], wr, experts, sh.k, bias, bias_mode, wl.act_mode)
    stream = torch.cuda.current_stream()

    def step(i, ev=None, mk=None):
        fw.set_x(xs[i % nbatch])
        if ev is None and mk is None:
            fw()  # k3moe_forward: the whole layer in one C call
        elif mk is None:
            # the same work as two calls, HIP events on this stream around
            # the expert-FFN stage (k3moe_ffn)
            fw.run_route()
            ev[0].record(stream)
            fw.run_ffn()
            ev[1].record(stream)
        else:
            # the same, every kernel of the stage timed by its own dispatch events
            fw.run_route()
            mk.set()
            try:
                fw.run_ffn()
            finally:
                k3.StageMarks.clear()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if use_graph:
        gx = xs[0].clone()
        fw.set_x(gx)
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            fw.stream = s
            fw()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            fw()
        fw.stream = None
        torch.cuda.synchronize()

    # timed region: K steps; event-marked steps carry events around their
    # expert-FFN stage.  An event record costs a few microseconds of stream
    # time, so one-token steps (~0.1 ms) are marked one in EV_EVERY_DECODE
    # (more often when there are fewer than MIN_EV_SAMPLES * EV_EVERY_DECODE).
    # Kernel marks (k3moe_set_stage_marks: each kernel of the stage launched
    # with its own start / end events, which add nothing to the stream) go on
    # other steps than the stage events when steps are short (so that the
    # stage interval holds no marked launch), on the same steps otherwise.
    ev_every = max(1, min(EV_EVERY_DECODE if T == 1 else 1, steps // MIN_EV_SAMPLES))
    nev = (steps + ev_every - 1) // ev_every
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    mk_off = ev_every // 2 if ev_every > 1 else 0
    nmk = len(range(mk_off, steps, ev_every)) if graph is None else 0
    mks = [k3.StageMarks(k3.MAX_MARKS, stream) for _ in range(nmk)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if graph is None:
        for i in range(steps):
            ev = evs[i // ev_every] if i % ev_every == 0 else None
            mk = mks[i // ev_every] if i % ev_every == mk_off else None
            if ev is not None and mk is not None:  # every step carries events: marks and stage together
                fw.set_x(xs[i % nbatch])
                fw.run_route()
                ev[0].record(stream)
                mk.set()
                try:
                    fw.run_ffn()
                finally:
                    k3.StageMarks.clear()
                ev[1].record(stream)
            else:
                step(i, ev, mk)
    else:
        for i in range(steps):
            gx.copy_(xs[i % nbatch], non_blocking=True)
            graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / steps
    tokens_per_s = T * steps / elapsed

    # bytes of the active experts, from this run's own counts (last step)
    counts = fw.route["counts"].cpu().numpy()
    n_active = int((counts > 0).sum())
    expert_bytes = n_active * sh.expert_bytes
    act_bytes = 2 * T * sh.d * 4  # x read, y written
    roofline = None
    if graph is None:
        ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        kern = kernel_times(mks)
        kb = kernel_bytes(sh, T, n_active, wl.act_mode)
        stage = {"kernels": "every kernel k3moe_ffn launches", "bytes_per_launch": expert_bytes + act_bytes,
                 "avg_ms": round(ffn_ms, 5), "event_samples": len(evs),
                 "achieved": round((expert_bytes + act_bytes) / (ffn_ms * 1e-3) / 1e9, 1),
                 "traffic": measured_traffic(wl.name)}
        stage["frac"] = round(stage["achieved"] / HBM_PEAK_GBS, 4)
        # the dominant kernel: the longest of the stage, timed by its marks
        dom = max((n for n in kern if kb.get(n)), key=lambda n: kern[n]["avg_ms"])
        per = {}
        for n, v in kern.items():
            b = kb.get(n)
            per[n] = {"avg_ms": round(v["avg_ms"], 5), "bytes_per_launch": b}
            if b:
                per[n]["frac"] = round(b / (v["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        achieved = kb[dom] / (kern[dom]["avg_ms"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name, KERNEL_NAMES[dom]),
                    "kernel": f"{dom} ({KERNEL_NAMES[dom]}*)", "bytes_per_launch": kb[dom],
                    "avg_ms": round(kern[dom]["avg_ms"], 5), "event_samples": len(mks),
                    "kernels": per, "stage": stage}
        # the whole layer per step (router weights + active experts + x, y) over the timed step time
        layer_bytes = sh.E * sh.d * 4 + expert_bytes + act_bytes
        roofline["layer"] = {"bytes_per_step": layer_bytes,
                             "frac": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if wl.act_mode == "mxfp4":
            flops = 2.0 * 3 * sh.d * sh.f * T * sh.k
            stage["flops_per_launch"] = flops
            stage["mfma_frac"] = round(flops / (ffn_ms * 1e-3) / 1e12 / MXFP4_PEAK_TFLOPS, 4)
            kf = {"gateup": 2.0 * 2 * sh.d * sh.f * T * sh.k, "down": 2.0 * sh.d * sh.f * T * sh.k}
            if dom in kf:
                tf = kf[dom] / (kern[dom]["avg_ms"] * 1e-3) / 1e12
                roofline["flops_per_launch"] = kf[dom]
                roofline["mfma_frac"] = round(tf / MXFP4_PEAK_TFLOPS, 4)
                # above the ridge (flop per byte over peak flops per peak byte) the matrix peak bounds it
                if kf[dom] / (MXFP4_PEAK_TFLOPS * 1e12) > kb[dom] / (HBM_PEAK_GBS * 1e9):
                    roofline.update({"bound": "mfma", "achieved": round(tf, 1), "peak": MXFP4_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": roofline["mfma_frac"],
                                     "hbm_frac": round(achieved / HBM_PEAK_GBS, 4)})
    return dict(fw=fw, xs=xs, nbatch=nbatch, stream=stream, ms_per_step=ms_per_step,
                tokens_per_s=tokens_per_s, roofline=roofline, n_active=n_active, bias_mode=bias_mode,
                graph=graph)


def measure_cache(k3, synthdata, torch, wl, experts, wr, xs, n_slots, steps):
    """Single-token decode through k3moe_forward_cached: every expert in
    pinned host memory, n_slots of them in HBM under the step-batched LRU.
    The cache is warmed with n_slots // k steps of other tokens, then `steps`
    fresh tokens are timed end to end (routing, policy, copies of the missed
    experts over the host link, expert FFN).  Hit rate from the device
    counters, checked against the oracle's LRU replay of the same selections,
    with Belady's optimum on that trace for comparison."""
    from oracle import cache as oc
    sh = wl.shape
    t0 = time.time()
    host = {}
    for w, (c, sc) in experts.items():
        hc = torch.empty(c.shape, dtype=torch.uint8, pin_memory=True)
        hs = torch.empty(sc.shape, dtype=torch.uint8, pin_memory=True)
        hc.copy_(c)
        hs.copy_(sc)
        host[w] = (hc, hs)
    torch.cuda.synchronize()
    log(f"host store pinned in {time.time() - t0:.1f}s")
    nx = len(xs)
    warm = max(1, n_slots // sh.k)
    cf = k3.CachedForward(xs[0], wr, host, n_slots, sh.k)
    for i in range(warm):
        cf.set_x(xs[(nx - 1 - i) % nx])
        cf()
    torch.cuda.synchronize()
    before = cf.read()
    t_start = time.perf_counter()
    for i in range(steps):
        cf.set_x(xs[i % nx])
        cf()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    after = cf.read()
    hits, misses = after["hits"] - before["hits"], after["misses"] - before["misses"]
    # the same selections replayed by the oracle (routing is deterministic)
    fr = k3.Forward(xs[0], wr, experts, sh.k)
    trace = []
    for i in list(range(warm)) + list(range(steps)):
        fr.set_x(xs[(nx - 1 - i) % nx] if len(trace) < warm else xs[i % nx])
        fr.run_route()
        trace.append(fr.route["topk_idx"].cpu().numpy().ravel().tolist())
    lru = oc.lru_replay(trace, n_slots)
    lru_h = sum(r["hits"] for r in lru[warm:])
    total_all = sum(r["hits"] + r["misses"] for r in lru)
    opt_h_all, _ = oc.opt_replay(trace, n_slots)
    ms = elapsed * 1e3 / steps
    miss_bytes = misses * sh.expert_bytes / steps
    del cf, fr, host
    return {"slots": n_slots, "hbm_bytes": n_slots * sh.expert_bytes, "host_store_bytes": sh.E * sh.expert_bytes,
            "policy": "step-batched LRU", "warmup_steps": warm, "steps": steps, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(1e3 / ms, 1), "hit_rate": round(hits / max(1, hits + misses), 4),
            "misses_per_step": round(misses / steps, 3), "host_link_bytes_per_step": round(miss_bytes),
            "host_link_GBps": round(miss_bytes / (ms * 1e-3) / 1e9, 2),
            "oracle_lru_hit_rate": round(lru_h / max(1, hits + misses), 4),
            "whole_trace": {"steps": len(trace), "lru_hit_rate": round(sum(r["hits"] for r in lru) / total_all, 4),
                            "belady_hit_rate": round(opt_h_all / total_all, 4)},
            "trace": "the timed tokens' own selections (uniform routing: no reuse beyond chance)"}


# mark kinds -> the kernel name prefix in the profiles
KERNEL_NAMES = {"active_list": "active_list", "quantize": "quantize_rows", "gateup": "gateup_",
                "down": "down_", "down_combine": "down_", "combine": "combine_"}


def kernel_times(mks):
    """Mean time of each kind of kernel of the stage over the marked steps
    (each kernel's own dispatch start to end; kernels of one kind in a step
    added up)."""
    acc = {}
    kinds = None
    for m in mks:
        ks = m.kinds()
        if kinds is None:
            kinds = ks
        if ks != kinds:
            raise RuntimeError(f"the stage launched different kernels across steps: {kinds} / {ks}")
        step = {}
        for i, n in enumerate(ks):
            step[n] = step.get(n, 0.0) + m.kernel_ms(i)
        for n, t in step.items():
            acc.setdefault(n, []).append(t)
    return {n: {"avg_ms": float(np.mean(v)), "samples": len(v)} for n, v in acc.items()}


def kernel_bytes(sh, T, n_active, act_mode):
    """Algorithmic bytes of each kernel of the stage: the active experts'
    weights it streams once, the activations it reads and the outputs it
    writes (h of the one-token path stays an on-chip intermediate of the
    method and is not counted)."""
    P, d, f = T * sh.k, sh.d, sh.f
    w_gu = n_active * 2 * f * (d // 2 + d // 32)
    w_dn = n_active * d * (f // 2 + f // 32)
    mx_row = lambda n: n // 2 + n // 32  # noqa: E731  MXFP4 bytes of n values
    if act_mode == "mxfp4":
        return {"active_list": None, "quantize": T * d * 4 + T * mx_row(d),
                "gateup": w_gu + T * mx_row(d) + P * mx_row(f),
                "down": w_dn + P * mx_row(f) + P * d * 4,
                "combine": P * d * 4 + T * d * 4}
    return {"active_list": None, "gateup": w_gu + T * d * 4, "down_combine": w_dn + T * d * 4,
            "down": w_dn + P * d * 4, "combine": P * d * 4 + T * d * 4}


def measured_traffic(workload, prefix=None):
    """HBM bytes per expert-FFN launch (or, with prefix, per launch of the
    stage's kernel whose name holds it) from the committed counter profile
    (FETCH_SIZE / WRITE_SIZE scaled by a plain-copy calibration), or None
    when the kernel sources changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != rec.get("source_sha") or workload not in rec.get("workloads", {}):
        return None
    w = rec["workloads"][workload]
    total = 0.0
    for name, v in w["kernels"].items():
        if (prefix in name) if prefix else any(key in name for key in FFN_KERNELS):
            total += (v["fetch_kib"] * w["fetch_scale"] + v["write_kib"] * w["write_scale"]) * 1024
    return round(total)


def cpu_baseline(sh, wl, budget_s):
    """The fp64 oracle, as it stands, on the host cores: whole layer (router
    over all experts, top-k, grouping, expert FFNs, combine) for as many
    tokens of the workload as fit the time budget (at least one).  Expert
    weights for the sampled tokens are generated before the clock starts."""
    import oracle
    import synthdata

    wr = synthdata.router_weight(sh)
    bias = synthdata.zipf_bias(sh) if wl.zipf_bias else None
    bm = oracle.BIAS_LOGITS if wl.zipf_bias else oracle.BIAS_NONE
    cache = {}
    done, spent, tok = 0, 0.0, 0
    while done == 0 or spent < budget_s:
        x = synthdata.tokens(sh, 1, first=tok)
        r = oracle.route(x, wr, sh.k, bias, bm)          # warm expert cache outside the clock
        for e in r["topk_idx"][0]:
            if int(e) not in cache:
                cache[int(e)] = synthdata.expert(sh, int(e))
        t0 = time.perf_counter()
        r = oracle.route(x, wr, sh.k, bias, bm)
        oracle.token_forward(x[0], r["topk_idx"][0], r["topk_w"][0], lambda e: cache[int(e)],
                             act_mode=wl.act_mode)
        spent += time.perf_counter() - t0
        done += 1
        tok += 1
        if len(cache) > 256:
            cache.clear()
    threads = oracle.num_threads()
    # one more token on a single thread, for context
    oracle.set_num_threads(1)
    x = synthdata.tokens(sh, 1, first=tok)
    r = oracle.route(x, wr, sh.k, bias, bm)
    for e in r["topk_idx"][0]:
        if int(e) not in cache:
            cache[int(e)] = synthdata.expert(sh, int(e))
    t0 = time.perf_counter()
    r = oracle.route(x, wr, sh.k, bias, bm)
    oracle.token_forward(x[0], r["topk_idx"][0], r["topk_w"][0], lambda e: cache[int(e)], act_mode=wl.act_mode)
    one_thread_s = time.perf_counter() - t0
    oracle.set_num_threads(threads)
    return {"value": round(done / spent, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} single tokens of {wl.name} (full layer per token, fp64), {spent:.1f}s",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "one_thread_s_per_token": round(one_thread_s, 3)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
