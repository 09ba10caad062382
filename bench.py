"""Benchmark of the routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (router, top-k, grouping, expert FFN on
MXFP4 weights, combine) over one batch of synthetic tokens already resident
in HBM.  The default workload is single-token greedy decode on the
896-expert / top-16 layer (d_model 7168, d_ff 2048), a fresh seeded token per
step (1000 distinct tokens, cycled).

Prints one JSON line: throughput in tokens/s, the expert-FFN stage against the
HBM roofline (active-expert bytes / the stage's average duration, timed with
HIP events on the launch stream), and the fp64 oracle timed on the host cores
on a bounded sample of the same workload.
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
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB three times "
                         "(reference kernel for hardware byte counters; not part of the step)")
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
    bias = torch.from_numpy(synthdata.zipf_bias(sh)).to(dev) if wl.zipf_bias else None
    bias_mode = "logits" if wl.zipf_bias else "none"
    # distinct seeded batches, resident in HBM before timing
    nbatch = 1000 if T == 1 else max(1, min(8, 1000 // T))
    xs = [torch.from_numpy(synthdata.tokens(sh, T, first=i * T)).to(dev) for i in range(nbatch)]
    torch.cuda.synchronize()
    log(f"inputs resident in {time.time() - t0:.1f}s ({nbatch} batches)")

    fw = k3.Forward(xs[0], wr, experts, sh.k, bias, bias_mode, wl.act_mode)
    stream = torch.cuda.current_stream()
    route = fw.route

    def step(i, ev=None):
        fw.set_x(xs[i % nbatch])
        if ev is None:
            fw()  # k3moe_forward: the whole layer in one C call
        else:
            # the same work as two calls, HIP events on this stream around
            # the expert-FFN stage (k3moe_ffn)
            fw.run_route()
            ev[0].record(stream)
            fw.run_ffn()
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
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
    # time, so one-token steps (~0.1 ms) are marked one in EV_EVERY_DECODE.
    EV_EVERY = EV_EVERY_DECODE if T == 1 else 1
    nev = (args.steps + EV_EVERY - 1) // EV_EVERY
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if graph is None:
        for i in range(args.steps):
            step(i, evs[i // EV_EVERY] if i % EV_EVERY == 0 else None)
    else:
        for i in range(args.steps):
            gx.copy_(xs[i % nbatch], non_blocking=True)
            graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed

    # bytes of the active experts, from this run's own counts (last step)
    counts = route["counts"].cpu().numpy()
    n_active = int((counts > 0).sum())
    expert_bytes = n_active * sh.expert_bytes
    act_bytes = 2 * T * sh.d * 4  # x read, y written
    roofline = None
    if graph is None:
        ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        achieved = (expert_bytes + act_bytes) / (ffn_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name),
                    "kernel": "expert FFN stage (every kernel k3moe_ffn launches; decode: gate/up GEMV "
                              "with SwiGLU + down GEMV with the fused combine)",
                    "bytes_per_launch": expert_bytes + act_bytes, "avg_ms": round(ffn_ms, 5)}
        # the whole layer per step (router weights + active experts + x, y) over the timed step time
        layer_bytes = sh.E * sh.d * 4 + expert_bytes + act_bytes
        roofline["layer"] = {"bytes_per_step": layer_bytes,
                             "frac": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if wl.act_mode == "mxfp4" and roofline is not None:
        flops = 2.0 * 3 * sh.d * sh.f * T * sh.k
        roofline["mfma_frac"] = round(flops / (roofline["avg_ms"] * 1e-3) / 1e12 / MXFP4_PEAK_TFLOPS, 4)

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
            dst.copy_(src)
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
    if flushed is not None:
        out["flushed"] = flushed
    print(json.dumps(out), flush=True)


def measured_traffic(workload):
    """HBM bytes per expert-FFN launch from the committed counter profile
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
        if any(key in name for key in FFN_KERNELS):
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
    return {"value": round(done / spent, 4), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} single tokens of {wl.name} (full layer per token, fp64), {spent:.1f}s"}


if __name__ == "__main__":
    main()
