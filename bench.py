"""Benchmark of the FP8 MoE feed-forward step on one MI355X.

Workload (one "step" = one forward of the whole path: route + quantise + FC13 + SwiGLU,
re-quantise + FC2, combine): the routed decode step at Maverick scale, M = 4 tokens
(one token plus a 3-token draft), hidden 5120, intermediate 8192, 128 routed experts
plus one shared expert, top-1 routing forced onto d = 4 distinct experts, FP8 e4m3
weights with per-channel scales, bf16 activations and output.

Cache defeat: two independent 129-expert weight pools (about 16 GB each) are
resident; consecutive steps alternate pools and rotate through 32 disjoint sets of
4 experts, so a routed expert's bytes are read again only after 64 steps (~40 GB of
traffic) and each pool's shared expert every second step (~1.1 GB apart), both far
beyond the 256 MB Infinity Cache.

Warm-up: the first visits of each of the 64 (pool, expert set) pairs run a few us
slower than later ones, and the step time settles after about three passes (a
serving process is in that steady state).  The default warm-up, 200 steps of the same
work as the timed ones, gets there; with 20 the timed steps come out 2-4 us slower.

Reported: us per step (plain stream launches through the C ABI, and the same K steps
replayed from one HIP graph; p10/p50/p90 from an event pair around each step), achieved
HBM GB/s of the step, the dominant kernel's roofline (FC13: algorithmic bytes / its
average duration from HIP events recorded on its stream over a timed region), the
matrix-instruction utilisation, the attainable read bandwidth measured by the library's
streaming-read probe, and the float64 CPU oracle timed on one step.

    python bench.py [--gpus 1] [--steps 200] [--warmup 200] [--no-cpu]
                    [--dense] [--m M] [--d D] [--zipf] [--pools P]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_F16_TFLOPS = 2500.0  # MI355X dense f16 matrix peak (the instruction the kernels use)
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "fc13_hbm_counters.json")
KERNEL_SOURCES = ("codec.hpp", "layout.hpp", "params.hpp", "prologue.hpp", "fc13.hpp")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp8_moe_ffn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--d", type=int, default=4, help="distinct routed experts per step")
    ap.add_argument("--pools", type=int, default=0,
                    help="independent weight pools (default 2; 8 for --dense, whose pool is one expert)")
    ap.add_argument("--variant", choices=["gate-on-input", "static-scales"], default=None,
                    help="a variant reading: the gate on the routed expert's input, or static "
                         "per-tensor scales for x and the intermediate (calibrated on the same inputs)")
    ap.add_argument("--rmsnorm", action="store_true",
                    help="the step with the RMSNorm in front fused into its first kernel (x is then "
                         "the hidden state; seeded norm weight, eps 1e-5)")
    ap.add_argument("--ceiling-gib", type=int, default=4,
                    help="GiB read by the streaming-read probe (the attainable HBM read bandwidth); 0: skip")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="end with 3 device-to-device copies of this many MiB: a plain copy of known "
                         "size, against which the HBM byte counters of a profiler run are scaled")
    ap.add_argument("--zipf", action="store_true",
                    help="Zipf(1.2) expert popularity instead of d forced experts (throughput batch)")
    ap.add_argument("--batch-mode", choices=["grouped", "chunked"], default="grouped",
                    help="how a batch above 8 tokens runs: grouped passes (every active expert read "
                         "once per pass) or launches of up to 16 tokens")
    ap.add_argument("--launch", choices=["three", "single"], default="three",
                    help="decode launches as three kernels, or as one kernel in three phases")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--dense", action="store_true", help="dense shared-expert FFN instead")
    ap.add_argument("--m", type=int, default=4)
    ap.add_argument("--inter", type=int, default=0,
                    help="intermediate size (default 8192); 1024 is one GPU's share of the FFN split "
                         "8 ways over I, with the intermediate's scale taken over the local share")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(no collectives or sharding are built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import fp8_moe_ffn_amd as F
    import workloads as W

    F.load()
    if args.pools <= 0:
        args.pools = 8 if args.dense else 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    K, I = W.HIDDEN, (args.inter or W.INTER)
    E = 0 if args.dense else W.EXPERTS
    M, d = args.m, (0 if args.dense else args.d)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)

    # ---- weights: `pools` independent pools of E routed + 1 shared expert -------------
    t0 = time.time()
    ffns = []
    for pool in range(args.pools):
        f = F.MoeFFN(K, I, E, M)
        f.set_batch_mode(F.BATCH_CHUNKED if args.batch_mode == "chunked" else F.BATCH_GROUPED)
        if args.launch == "single":
            f.set_launch_mode(F.LAUNCH_SINGLE)
        for slot in range(E + 1):
            e = W.expert(pool, slot, K, I, dev)
            f.prepack_expert(slot, e.w13, e.s13, e.w2, e.s2)
            del e
        ffns.append(f)
        log(f"pool {pool}: {E + 1} experts packed ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    x = W.activations(0, M, K, dev)
    out = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    rot = []  # forced routings, 4 distinct experts each, disjoint across the rotation
    if E and args.zipf:  # 8 seeded Zipf(1.2) batches
        base = W.router_logits(0, M, E, dev)
        for r in range(8):
            rot.append(W.force_routing(base, W.zipf_targets(r, M, E)).contiguous())
        d = float(np.mean([len(set(W.zipf_targets(r, M, E))) for r in range(8)]))  # the steps cycle the 8
    elif E:
        perm = np.random.default_rng(1234).permutation(E)
        nrot = E // d
        base = W.router_logits(0, M, E, dev)
        for r in range(nrot):
            tg = [int(perm[r * d + (m % d)]) for m in range(M)]
            rot.append(W.force_routing(base, tg).contiguous())
    else:
        rot = [None]
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    xp, op = x.data_ptr(), out.data_ptr()
    lps = [r.data_ptr() if r is not None else None for r in rot]

    variant = None
    if args.variant == "gate-on-input":
        variant = F.Variant(1, 0.0, 0.0)
    elif args.variant == "static-scales":
        # calibration: one per-tensor scale each, the largest dynamic scale of the inputs
        # over the rotation (a debug forward of each expert set gives the intermediate's)
        dbg = F.debug_buffers(M, K, I, dev)
        sx_max = sa_max = 0.0
        for r in rot:
            ffns[0].forward_debug(x, r, out, dbg)
            torch.cuda.synchronize()
            sx_max = max(sx_max, float(dbg.s_x.max()))
            sa_max = max(sa_max, float(dbg.s_a_shared.max()), float(dbg.s_a_routed.max()) if E else 0.0)
        variant = F.Variant(0, sx_max, sa_max)
        log(f"static scales: x {sx_max:.6g}, intermediate {sa_max:.6g}")

    norm_w = W.norm_weight(0, K, dev) if args.rmsnorm else None

    def forward(f, lp, stream_handle):
        if norm_w is not None:
            return f.forward_rmsnorm_raw(xp, norm_w.data_ptr(), 1e-5, lp, op, M, stream_handle, variant)
        if variant is None:
            return f.forward_raw(xp, lp, op, M, stream_handle)
        return f.forward_variant_raw(xp, lp, op, M, stream_handle, variant)

    def step(i):
        f = ffns[i % len(ffns)]
        lp = lps[(i // len(ffns)) % len(lps)]
        st = forward(f, lp, sh)
        if st != F.OK:
            raise F.MoeError(st, "forward")

    # ---- plain stream launches ---------------------------------------------------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    us_stream = ev0.elapsed_time(ev1) * 1e3 / args.steps
    log(f"stream launches: {us_stream:.2f} us/step (host wall {wall / args.steps * 1e6:.2f} us/step)")

    # ---- the same steps, one event pair each: the distribution -------------------------
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        pairs[i][0].record(stream)
        step(i)
        pairs[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    pct = {f"p{q}": round(float(np.percentile(per_step, q)), 3) for q in (10, 50, 90)}
    log(f"per-step events: p10 {pct['p10']:.2f}  p50 {pct['p50']:.2f}  p90 {pct['p90']:.2f} us")

    # ---- HIP graph replay: the same K steps captured into one graph -------------------
    # (a serving loop puts its whole iteration into one graph; each graph launch costs a
    # fixed gap before its first kernel on this runtime, about 8 us measured, and nothing
    # between the kernels inside it, so a graph of one step would time that gap instead)
    g = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            for i in range(args.steps):
                f = ffns[i % len(ffns)]
                lp = lps[(i // len(ffns)) % len(lps)]
                st = forward(f, lp, gs.cuda_stream)
                assert st == F.OK
    torch.cuda.synchronize()
    for _ in range(max(1, -(-args.warmup // args.steps))):  # at least W steps of warm-up
        g.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_graph = ev0.elapsed_time(ev1) * 1e3 / args.steps
    log(f"graph replay ({args.steps} steps in one graph): {us_graph:.2f} us/step")
    del g

    # ---- per-kernel durations over a timed region (HIP events on the launch stream) ----
    for f in ffns:
        f.profile_begin()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    stage_ms = [0.0] * F.NUM_STAGES
    calls = 0
    for f in ffns:
        ms, c = f.profile_end()
        stage_ms = [a + b for a, b in zip(stage_ms, ms)]
        calls += c
    # (forwards of more than one launch of tokens are not recorded per kernel)
    stage_us = {n: stage_ms[k] * 1e3 / calls for k, n in enumerate(F.STAGE_NAMES)} if calls else {}
    if args.launch == "single" and stage_us:  # one kernel: the events bracket it whole
        stage_us = {"single": sum(stage_us.values())}
    log("per-kernel us: " + ", ".join(f"{k} {v:.2f}" for k, v in stage_us.items()))

    # ---- bytes --------------------------------------------------------------------------
    S = 1 + d
    w13_bytes = K * 2 * I + 2 * I * 4  # codes + scales of one expert's FC13
    w2_bytes = I * K + K * 4
    step_bytes = round(S * (w13_bytes + w2_bytes) + M * K * 2 * 2 + M * E * 2)  # + x, out, logits
    # FC13 moves the codes and scales of S experts, reads x and the logits (its prologue
    # routes and quantises), writes the float32 intermediate a [2M][I]
    fc13_bytes = round(S * w13_bytes + M * K * 2 + M * E * 2 + (2 * M if E else M) * I * 4)
    if args.rmsnorm:  # the norm weight
        fc13_bytes += K * 2
        step_bytes += K * 2
    us_best = min(us_stream, us_graph)
    # matrix work: 2 (K 2I + I K) flops per (token, expert) pair; each token meets the
    # shared expert and, with routed experts, one more
    pair_flops = 2 * (K * 2 * I + I * K)
    flops = pair_flops * M * (2 if E else 1)
    mfma_tflops = flops / (us_best * 1e-6) / 1e12
    fc13_us = stage_us.get("fc13_swiglu", float("nan"))
    if args.launch == "single":  # the dominant kernel is the whole step
        fc13_us, fc13_bytes = stage_us.get("single", float("nan")), step_bytes
    achieved = fc13_bytes / (fc13_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        with open(PROFILE_COUNTERS) as fh:
            pc = json.load(fh)
        if (pc.get("kernel_hash") == kernel_hash() and pc.get("workload") == ("dense" if args.dense else "routed")
                and args.variant is None and not args.rmsnorm and args.launch == "three"):  # the plain kernel
            traffic = pc.get("traffic_bytes_per_launch")

    res = {
        "metric": "\u00b5s per M=4 MoE-FFN step + achieved HBM GB/s (% of MI355X peak)"
                  if M == 4 else f"\u00b5s per M={M} MoE-FFN step + achieved HBM GB/s (% of MI355X peak)",
        "value": round(us_best, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_best / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)",
        "data": "synthetic, seeded (weights 0.02*N(0,1) per-channel e4m3; x, logits bf16 N(0,1))",
        "config": {
            "variant": args.variant,
            "fused_rmsnorm": bool(args.rmsnorm),
            "batch_mode": (args.batch_mode if M > F.GROUP_FROM else None),
            "launch": args.launch,
            "workload": ("dense shared-expert FFN" if args.dense else
                         f"routed MoE FFN, Zipf(1.2) popularity, {d:.3f} distinct of {E} experts + shared (mean)"
                         if args.zipf else
                         f"routed MoE FFN decode step, {d} distinct of {E} experts + shared"),
            "M": M, "hidden": K, "inter": I, "num_experts": E, "distinct_active": d,
            "weight_pools": len(ffns), "rotation_sets": len(lps),
        },
        "us_per_step_stream": round(us_stream, 3),
        "us_per_step_graph": round(us_graph, 3),
        "step_bytes": step_bytes,
        "hbm_GBps": round(step_bytes / (us_best * 1e-6) / 1e9, 1),
        "hbm_frac_of_peak": round(step_bytes / (us_best * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "us_per_step_events": pct,
        "stage_us": {k: round(v, 3) for k, v in stage_us.items()},
        "mfma": {
            "instruction": "v_mfma_f32_16x16x32_f16 (e4m3 codes widened exactly to f16)",
            "flops_per_step": flops,
            "achieved_TFLOPs": round(mfma_tflops, 2),
            "peak_TFLOPs": PEAK_F16_TFLOPS,
            "util": round(mfma_tflops / PEAK_F16_TFLOPS, 5),
        },
        "roofline": {
            "kernel": "single_kernel" if args.launch == "single" else "fc13_swiglu_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1) if stage_us else None,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4) if stage_us else None,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": fc13_bytes,
            "avg_launch_us": round(fc13_us, 3) if stage_us else None,
        },
    }

    # ---- attainable read bandwidth (streaming-read probe over a large buffer) ----------
    if args.ceiling_gib > 0:
        buf = torch.empty(args.ceiling_gib << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(2):
            F.stream_read(buf, sink)
        ev0.record(stream)
        reps = 5
        for _ in range(reps):
            F.stream_read(buf, sink)
        ev1.record(stream)
        torch.cuda.synchronize()
        ceil_gbps = buf.numel() * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
        del buf
        res["ceiling"] = {"kernel": "stream_read (C ABI probe)", "bytes": args.ceiling_gib << 30,
                          "GBps": round(ceil_gbps, 1), "frac_of_peak": round(ceil_gbps / PEAK_HBM_GBPS, 4)}
        res["hbm_frac_of_ceiling"] = round(res["hbm_GBps"] / ceil_gbps, 4)
        log(f"streaming-read ceiling: {ceil_gbps:.1f} GB/s; step at {res['hbm_frac_of_ceiling']:.3f} of it")

    # ---- CPU oracle baseline -------------------------------------------------------------
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(args, x, rot[0], E, K, I, M, dev)

    print(json.dumps(res), flush=True)
    for f in ffns:
        f.close()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {n} bytes")


def cpu_baseline(args, x, logits, E, K, I, M, dev):
    """The float64 oracle on one step of the same workload (pool 0, first expert set):
    weights of the touched experts are generated, copied to the host and excluded
    from the timing; repeated until --cpu-seconds of CPU time, median reported."""
    import numpy as np
    import workloads as W
    from oracle import ffn as oracle_ffn

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    xb = W.bits(x)
    lb = W.bits(logits) if logits is not None else None
    need = [E]
    if E:
        need += sorted(set(int(e) for e in np.argmax(
            __import__("oracle").fp8.bf16_to_f64(lb), axis=1)))
    cache = {s: W.expert(0, s, K, I, dev).numpy() for s in need}

    def timed(budget, max_runs):
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle_ffn.forward(xb, lb, cache.__getitem__, E)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget or len(times) >= max_runs:
                return float(np.median(times)) * 1e6, len(times)

    us, runs = timed(args.cpu_seconds, 5)
    one = None
    try:  # the same with the BLAS held to one thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            us1, runs1 = timed(args.cpu_seconds, 3)
        one = {"value": round(us1, 1), "unit": "us/step", "cores": 1, "runs": runs1}
    except ImportError:
        pass
    return {"value": round(us, 1), "unit": "us/step", "kind": "oracle",
            "cores": blas_threads if blas_threads else os.cpu_count(),
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "runs": runs,
            "single_thread": one,
            "sample": f"one full step (M={M}, {len(need) - 1} routed + shared experts), "
                      "weights already on the host, median of the runs"}


if __name__ == "__main__":
    main()
