#!/usr/bin/env python3
"""Benchmark of the block-diffusion denoising round on one MI355X.

A step is one full round on a 32-position block: RMSNorm, router and top-8 of
256 experts, union-of-experts SwiGLU plus the shared expert and the weighted
combine (one Clover-shaped MoE layer: hidden 2048, intermediate 512, flat
routing, no coreset), the final RMSNorm, the LM head over a 248320-token
vocabulary with the fused softmax-confidence/argmax, and the LowConfidence
commit.  Inputs are seeded synthetic tensors, resident in HBM before timing.

Prints one JSON line: microseconds per round (K calls of
bdd_block_denoise_round on one stream, timed with events at the ends of the
region; the same K rounds replayed as HIP graphs are reported beside it),
achieved HBM bandwidth on the round's algorithmic bytes, the roofline of the
dominant kernel (its launches bracketed by hipEvents on their stream over K
further rounds; HBM traffic from the rocprofv3 counter summary under
profiles/ while the kernel's sources are unchanged since it was taken), the
same LM head with 4-bit weights timed alone ('lmhead_int4', not the value),
the 40-layer Zipf/coreset stack round with block resolves through the
generation driver ('stack', not the value), and the CPU oracle timed on a
bounded sample of the same workload (all host threads, then one).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--stack L]
                                             # (--stack 0 skips the 40-layer Zipf/coreset stack)
    python bench.py --int4-only              # the 4-bit LM head + commit alone
    python bench.py --copy-calibration MIB   # plain device copy, for counter scaling
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per 32-token block-denoise round; achieved HBM GB/s & % of roofline"
HBM_PEAK_GBPS = 8000.0
WORKLOAD = ("clover_block_round: 1 MoE layer (hidden 2048, 256 routed experts top-8, expert "
            "intermediate 512, shared expert 512, flat routing, no coreset) + final RMSNorm + LM head "
            "(vocab 248320) + LowConfidence commit (threshold 0.95), block 32, bf16 weights / fp32 accumulate")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (counter scaling)")
    ap.add_argument("--stack", type=int, default=40, metavar="L",
                    help="also measure an L-layer stack round (Zipf routing, coreset 0.9) and block resolves "
                         "on it; reported under 'stack', not as the value (0: skip)")
    ap.add_argument("--stack-only", type=int, default=0, metavar="L",
                    help="only run the L-layer stack measurement (for a kernel trace of that workload alone); "
                         "prints one JSON line with the 'stack' object")
    ap.add_argument("--int4-stack", type=int, default=40, metavar="L",
                    help="also measure the L-layer stack with 4-bit experts and LM head; reported under "
                         "'stack_int4' (0: skip)")
    ap.add_argument("--int4-stack-only", type=int, default=0, metavar="L",
                    help="only run the 4-bit L-layer stack measurement; prints one JSON line with 'stack_int4'")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the block-size / threshold sweep (T in 8, 16, 32, 64; threshold 0.8 .. 0.99) of "
                         "block resolves on the round stub; prints one JSON line per (T, threshold)")
    ap.add_argument("--int4-only", action="store_true",
                    help="only measure the 4-bit LM head + commit (for a kernel trace of it alone); prints one "
                         "JSON line with the 'lmhead_int4' object")
    ap.add_argument("--counter-run", nargs="?", const="flat", default=None, choices=["flat", "zipf", "int4"],
                    help="only run 3 rounds on inputs drawn with torch.randn (a handful of kernel launches "
                         "besides the library's), for hardware-counter collection: one Clover layer with flat "
                         "routing (flat), with Zipf router bias and the coreset at top_p 0.9 (zipf), or the "
                         "latter with 4-bit experts and LM head (int4)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_diffusion_decode_amd as bdd
    import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # a streaming copy kernel of known size (negation: one fp32 read and
        # one fp32 write per element) whose counter readings scale the
        # hardware counters to bytes
        n = args.copy_calibration << 20
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}), flush=True)
        return
    d = W.C1
    if args.sweep:
        sweep(args, W.C1, dev)
        return
    if args.stack_only:
        args.stack = args.stack_only
        print(json.dumps({"stack": stack_round(args, W.C1, dev)}), flush=True)
        return
    if args.int4_stack_only:
        args.int4_stack = args.int4_stack_only
        print(json.dumps({"stack_int4": stack_round(args, W.C1, dev, int4=True)}), flush=True)
        return
    if args.counter_run:
        counter_run(d, dev, args.counter_run)
        return
    if args.int4_only:
        print(json.dumps({"lmhead_int4": lmhead_int4(args, d, dev)}), flush=True)
        return
    R = 8
    log(f"[bench] generating inputs (seed {args.seed})")
    x, info = W.planted_round_inputs(args.seed, d, rounds=R, p=0.3, amp_pass=24.0, amp_fail=(10.0, 14.0))
    x = x.to(dev)
    layer = W.layer_weights(args.seed, 0, d, device=dev)
    w_lm = W.lm_head_weight(args.seed, d, device=dev, unit_rows=info["unit_rows"])
    dims = bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, bdd.BDD_BF16)
    lm = bdd.pack_lm_head(w_lm)
    plan = bdd.RoundPlan(dims, [layer], lm, 1.0, 0.95)
    T = d.T
    tok = torch.full((T,), bdd.MASK, dtype=torch.int32, device=dev)
    conf = torch.empty(T, dtype=torch.float32, device=dev)
    choice = torch.empty(T, dtype=torch.int32, device=dev)
    ri = torch.empty(4, dtype=torch.int32, device=dev)
    nd = torch.empty((R, 1), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    # distinct experts of each stub round (the GPU's own routing)
    for r in range(R):
        plan(x[r], tok, conf, choice, ri, None, nd[r])
    torch.cuda.synchronize()
    n_distinct = nd[:, 0].cpu().numpy().astype(np.int64)

    # one captured round per stub input (HIP graphs): a decode loop replays them
    graphs = [bdd.RoundGraph(plan, x[r], tok, conf, choice, ri) for r in range(R)]

    # warmup, with every kernel timed (eager) to find the dominant one
    bdd.timing_enable(True, None)
    for i in range(args.warmup):
        plan(x[i % R], tok, conf, choice, ri)
    torch.cuda.synchronize()
    warm = bdd.timing_read()
    bdd.timing_enable(False)
    dominant = max(warm, key=lambda k: warm[k][0])
    log("[bench] warmup per-kernel avg us: " +
        ", ".join(f"{k}={1e3 * v[0] / v[1]:.1f}" for k, v in warm.items()))
    for i in range(args.warmup):
        graphs[i % R].launch()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            fn(i)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps, time.perf_counter() - t0

    # timed region: K rounds through the C ABI, events only at its two ends;
    # then the same K rounds as graph replays
    ms, wall = timed(lambda i: plan(x[i % R], tok, conf, choice, ri))
    log(f"[bench] {args.steps} rounds: {ms * 1e3:.1f} us/round (host wall {wall * 1e3 / args.steps:.1f} us/round)")
    ms_graph, _ = timed(lambda i: graphs[i % R].launch())
    log(f"[bench] {args.steps} rounds (graph replays): {ms_graph * 1e3:.1f} us/round")
    spread = round_spread(args, lambda i: plan(x[i % R], tok, conf, choice, ri), stream)
    log(f"[bench] per-round events: median {spread['median']} us, p10 {spread['p10']}, p90 {spread['p90']}")

    # dominant kernel: K more rounds with its launches bracketed by hipEvents
    # on the stream it runs on
    bdd.timing_enable(True, dominant)
    timed(lambda i: plan(x[i % R], tok, conf, choice, ri))
    dom = bdd.timing_read()
    bdd.timing_enable(False)

    # algorithmic bytes: union experts + shared expert + router + LM head + block activations
    eb = 3 * d.H * d.I * 2
    mean_u = float(np.mean([n_distinct[i % R] for i in range(args.steps)]))
    lm_bytes = d.V * d.H * 2 + T * d.H * 2
    round_bytes = mean_u * eb + 3 * d.H * d.I_s * 2 + d.E * d.H * 2 + lm_bytes + T * d.H * 4 * 2
    gbps = round_bytes / (ms * 1e-3) / 1e9

    dom_ms = dom[dominant][0] / dom[dominant][1]
    dom_bytes = {"lmhead": lm_bytes,
                 "expert_gateup": (mean_u * d.I + d.I_s) * 2 * d.H * 2,
                 "expert_down": (mean_u * d.I + d.I_s) * d.H * 2}.get(dominant)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9 if dom_bytes else None
    traffic, traffic_src = measured_traffic(dominant)
    roofline = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS if achieved else None,
                "traffic": traffic, "avg_us": dom_ms * 1e3, "algorithmic_bytes": dom_bytes,
                "launches_timed": dom[dominant][1], "traffic_source": traffic_src}

    out = {
        "metric": METRIC,
        "value": round(ms * 1e3, 2),
        "unit": "us/round",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded counter-based inputs, random-init weights of the Clover shape",
        "config": {"workload": WORKLOAD, "global_batch": T, "seq_len": T, "parallelism": "single GPU",
                   "launch": "bdd_block_denoise_round per round on one stream",
                   "distinct_experts_mean": mean_u},
        "us_per_round_graph": round(ms_graph * 1e3, 2),
        "us_per_round_spread": spread,
        "round_bytes": round_bytes,
        "hbm_gbps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "per_kernel_warmup_us": {k: 1e3 * v[0] / v[1] for k, v in warm.items()},
        "roofline": roofline,
    }

    out["lmhead_int4"] = lmhead_int4(args, d, dev)
    out["lmhead_int4"]["bf16_lmhead_us_same_run"] = roofline["avg_us"]
    if args.stack > 0:
        del graphs, plan, lm, layer
        torch.cuda.empty_cache()
        out["stack"] = stack_round(args, d, dev)
        torch.cuda.empty_cache()
    if args.int4_stack > 0:
        out["stack_int4"] = stack_round(args, d, dev, int4=True)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, d, x, W.layer_weights(args.seed, 0, d, device=dev), w_lm, info,
                                           args.cpu_seconds)
    print(json.dumps(out), flush=True)


def round_spread(args, fn, stream, reps=None):
    """Median, p10 and p90 of single rounds, each bracketed by its own pair of
    events on the launch stream (a separate pass after the timed region)."""
    import numpy as np
    import torch

    reps = max(50, args.steps) if reps is None else reps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([1e3 * a.elapsed_time(b) for a, b in evs])
    return {"reps": reps, "median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2)}


def stack_round(args, d, dev, int4=False):
    """An L-layer stack of independent Clover-shaped layers (Zipf router bias,
    block coreset top_p 0.9, identity mixer) + LM head + commit: microseconds
    per round over K rounds of stub inputs (and the spread of single rounds),
    the distinct experts each layer read, and one block resolved from
    all-MASK by the generation driver (wall clock, host included).  With
    int4, every expert matrix (routed and shared) and the LM head are 4-bit
    (router bf16)."""
    import numpy as np
    import torch

    import block_diffusion_decode_amd as bdd
    import workloads as W

    L, top_p, T = (args.int4_stack if int4 else args.stack), 0.9, d.T
    log(f"[bench] {'4-bit ' if int4 else ''}stack: generating {L} layers")
    R = 32
    x, info = W.planted_round_inputs(args.seed, d, rounds=R, p=0.3, amp_pass=40.0, amp_fail=(14.0, 22.0),
                                     tag="stack")
    x = x.to(dev)
    if int4:
        layers = []
        for l in range(L):
            w = W.layer_weights_int4(args.seed, l, d, device=dev, bias="zipf", gamma=1.0)
            layers.append({"w_router": w["w_router"], "router_bias": w["router_bias"],
                           "w_gate_up": bdd.pack_int4(w["gu_codes"], w["gu_scales"]),
                           "w_down": bdd.pack_int4(w["dn_codes"], w["dn_scales"]),
                           "ws_gate_up": bdd.pack_int4(w["sgu_codes"], w["sgu_scales"]),
                           "ws_down": bdd.pack_int4(w["sdn_codes"], w["sdn_scales"])})
            del w
        codes, scales = W.lm_head_int4(args.seed, d, device=dev, unit_rows=info["unit_rows"])
        lm = bdd.pack_lm_head_int4(codes, scales)
        del codes, scales
        wdt = bdd.BDD_INT4
    else:
        layers = [W.layer_weights(args.seed, l, d, device=dev, bias="zipf", gamma=1.0) for l in range(L)]
        w_lm = W.lm_head_weight(args.seed, d, device=dev, unit_rows=info["unit_rows"])
        lm = bdd.pack_lm_head(w_lm)
        del w_lm
        wdt = bdd.BDD_BF16
    torch.cuda.empty_cache()
    plan = bdd.RoundPlan(bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, wdt), layers, lm, top_p, 0.95)
    tok = torch.full((T,), bdd.MASK, dtype=torch.int32, device=dev)
    conf = torch.empty(T, dtype=torch.float32, device=dev)
    choice = torch.empty(T, dtype=torch.int32, device=dev)
    ri = torch.empty(4, dtype=torch.int32, device=dev)
    nd = torch.empty((R, L), dtype=torch.int32, device=dev)
    for r in range(R):
        plan(x[r], tok, conf, choice, ri, None, nd[r])
    torch.cuda.synchronize()
    distinct = nd.cpu().numpy().astype(np.int64)
    # the same rounds without the coreset: the experts the coreset saves
    plan1 = bdd.RoundPlan(plan.d, layers, plan.lm, 1.0, 0.95)
    nd1 = torch.empty((R, L), dtype=torch.int32, device=dev)
    for r in range(R):
        plan1(x[r], tok, conf, choice, ri, None, nd1[r])
    torch.cuda.synchronize()
    distinct1 = nd1.cpu().numpy().astype(np.int64)
    del plan1
    steps = max(1, min(args.steps, 50))
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        plan(x[i % R], tok, conf, choice, ri)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    # per-kernel averages over a few more rounds (each launch bracketed by events)
    bdd.timing_enable(True, None)
    for i in range(8):
        plan(x[i % R], tok, conf, choice, ri)
    torch.cuda.synchronize()
    per_kernel = {k: round(1e3 * v[0] / v[1], 2) for k, v in bdd.timing_read().items()}
    bdd.timing_enable(False)
    mean_u = float(np.mean([distinct[i % R].sum() for i in range(steps)]))
    # algorithmic bytes: the union experts, the shared experts, the routers and
    # the LM head; a 4-bit matrix of n weights is n / 2 bytes of codes plus a
    # bf16 scale per 128 weights
    mat = (lambda n: n // 2 + n // 128 * 2) if int4 else (lambda n: 2 * n)
    eb = mat(3 * d.H * d.I)
    round_bytes = mean_u * eb + L * (mat(3 * d.H * d.I_s) + d.E * d.H * 2) + mat(d.V * d.H)
    spread = round_spread(args, lambda i: plan(x[i % R], tok, conf, choice, ri), torch.cuda.current_stream(),
                          reps=max(20, steps))
    # one block from all-MASK (round r takes stub r) through the generation
    # driver: the host one round ahead (the default), a host read after every
    # round, and all rounds enqueued with one read per block
    resolve = {}
    for mode, per_read in (("lookahead", 0), ("read_per_round", 1), ("one_read_per_block", R)):
        xr = x.reshape(1, R, T, d.H)
        bdd.generate(plan, xr, max_new_tokens=T, max_steps=R, eos_token=-7, rounds_per_read=per_read)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, rounds, _, stop, fbs = bdd.generate(plan, xr, max_new_tokens=T, max_steps=R, eos_token=-7,
                                                   rounds_per_read=per_read, with_fallbacks=True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        resolve[mode] = {"rounds": rounds[0], "fallback_rounds": fbs[0], "ms": round(1e3 * wall, 3),
                         "committed_tokens_per_s": round(T / wall, 1)}
    rounds, fallbacks = resolve["lookahead"]["rounds"], resolve["lookahead"]["fallback_rounds"]
    res = {"layers": L, "weights": "int4 experts and LM head, bf16 router" if int4 else "bf16",
           "coreset_top_p": top_p, "us_per_round": round(ms * 1e3, 2),
           "us_per_round_spread": spread,
           "distinct_experts_per_layer_mean": mean_u / L, "round_bytes": round_bytes,
           "hbm_gbps": round_bytes / (ms * 1e-3) / 1e9, "hbm_frac": round_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "per_kernel_launch_us": per_kernel,
           "distinct_experts_per_layer_without_coreset": float(distinct1.sum(axis=1).mean()) / L,
           "expert_bytes_saved_per_round": float((distinct1.sum(axis=1) - distinct.sum(axis=1)).mean()) * eb,
           "resolve": resolve}
    log(f"[bench] {'4-bit ' if int4 else ''}stack {L} layers: {ms * 1e3:.1f} us/round, {mean_u / L:.1f} experts/layer, "
        f"{res['hbm_gbps']:.0f} GB/s; block resolved in {rounds} rounds ({fallbacks} fallback), "
        f"{resolve['lookahead']['committed_tokens_per_s']:.0f} tok/s with the host one round ahead, "
        f"{resolve['read_per_round']['committed_tokens_per_s']:.0f} with a read per round, "
        f"{resolve['one_read_per_block']['committed_tokens_per_s']:.0f} with one read per block")
    return res


def sweep(args, d1, dev, blocks=4):
    """Block size and threshold sweep on the round stub: for each T the C1
    layer and LM head shapes with a T-position block, `blocks` blocks resolved
    from all-MASK round by round (stub round r feeds round r), for each
    threshold.  Reports rounds per block, fallback rounds, microseconds per
    round, algorithmic bytes per committed token and committed tokens/s."""
    import dataclasses

    import numpy as np
    import torch

    import block_diffusion_decode_amd as bdd
    import workloads as W

    for T in (8, 16, 32, 64):
        d = dataclasses.replace(d1, name=f"sweep_T{T}", T=T)
        dims = bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, bdd.BDD_BF16)
        layer = W.layer_weights(args.seed, 0, d, device=dev)
        xs, rows = [], set()
        for b in range(blocks):
            # failing peaks spread over amplitudes 12 .. 22, so confidences of
            # the not-passing positions cover the swept thresholds
            x, info = W.planted_round_inputs(args.seed, d, rounds=T, p=0.3, amp_pass=24.0,
                                             amp_fail=(12.0, 22.0), tag=f"sweep{b}")
            xs.append(x.to(dev))
            rows.update(int(v) for v in info["unit_rows"])
        w_lm = W.lm_head_weight(args.seed, d, device=dev, unit_rows=sorted(rows))
        lm = bdd.pack_lm_head(w_lm)
        del w_lm
        for tau in (0.8, 0.9, 0.95, 0.99):
            plan = bdd.RoundPlan(dims, [layer], lm, 1.0, tau)
            tok = torch.empty(T, dtype=torch.int32, device=dev)
            conf = torch.empty(T, dtype=torch.float32, device=dev)
            choice = torch.empty(T, dtype=torch.int32, device=dev)
            ri = torch.empty(4, dtype=torch.int32, device=dev)
            nd = torch.empty(1, dtype=torch.int32, device=dev)
            rounds, fallbacks, dist, ms_total = [], [], [], 0.0
            for b in range(blocks):
                tok.fill_(bdd.MASK)
                n = fb = 0
                t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t0.record()
                for r in range(T):
                    plan(xs[b][r], tok, conf, choice, ri, None, nd)
                    info_r = ri.cpu().tolist()
                    dist.append(int(nd.item()))
                    n += 1
                    fb += info_r[1]
                    if info_r[3]:
                        break
                t1.record()
                torch.cuda.synchronize()
                ms_total += t0.elapsed_time(t1)
                rounds.append(n)
                fallbacks.append(fb)
            # device time per round on the same rounds, without the host read between rounds
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for r in range(T):
                plan(xs[0][r], tok, conf, choice, ri)
            stop.record()
            torch.cuda.synchronize()
            us_round = 1e3 * start.elapsed_time(stop) / T
            eb = 3 * d.H * d.I * 2
            round_bytes = float(np.mean(dist)) * eb + 3 * d.H * d.I_s * 2 + d.E * d.H * 2 + d.V * d.H * 2
            mean_rounds = float(np.mean(rounds))
            res = {"sweep": {"T": T, "threshold": tau, "blocks": blocks, "rounds_per_block": mean_rounds,
                             "fallback_rounds_per_block": float(np.mean(fallbacks)),
                             "us_per_round": round(us_round, 2),
                             "bytes_per_committed_token": round_bytes * mean_rounds / T,
                             "committed_tokens_per_s_device": T / (mean_rounds * us_round * 1e-6),
                             "committed_tokens_per_s_with_host_reads": blocks * T / (ms_total * 1e-3),
                             "distinct_experts_mean": float(np.mean(dist))}}
            log(f"[bench] sweep T={T} threshold={tau}: {mean_rounds:.2f} rounds/block "
                f"({np.mean(fallbacks):.2f} fallback), {us_round:.1f} us/round, "
                f"{res['sweep']['bytes_per_committed_token'] / 1e6:.1f} MB per committed token")
            print(json.dumps(res), flush=True)
            del plan
        del lm, layer
        torch.cuda.empty_cache()


def counter_run(d, dev, mode="flat"):
    """Three rounds of the benchmark's shape on torch.randn inputs.  The bytes
    each kernel moves do not depend on the values beyond the routing (the LM
    head streams its whole weight either way), and the seeded counter
    generator's thousands of small launches stay out of the profiled process.
    mode: flat routing (flat); Zipf router bias with the coreset at top_p 0.9
    (zipf); the latter with 4-bit expert matrices and LM head (int4)."""
    import torch

    import block_diffusion_decode_amd as bdd
    import workloads as W

    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16

    def rnd(shape, std):
        return (torch.randn(shape, generator=g, device=dev) * std).to(bf)

    def i4(n, rows, cols, std):
        codes = torch.randint(0, 256, (n, rows, cols // 2), generator=g, device=dev, dtype=torch.uint8)
        scales = (torch.rand((n, rows, cols // 128), generator=g, device=dev) * 0.4 + 0.8) * (std / 2.5)
        return bdd.pack_int4(codes, scales.to(bf))

    bias = W.zipf_router_bias(0, 0, d.E).to(dev) if mode != "flat" else torch.zeros(d.E, device=dev)
    top_p = 0.9 if mode != "flat" else 1.0
    if mode == "int4":
        layer = {"w_router": rnd((d.E, d.H), d.w_std), "router_bias": bias,
                 "w_gate_up": i4(d.E, 2 * d.I, d.H, d.w_std), "w_down": i4(d.E, d.H, d.I, d.w_std),
                 "ws_gate_up": i4(1, 2 * d.I_s, d.H, d.w_std), "ws_down": i4(1, d.H, d.I_s, d.w_std)}
        codes = torch.randint(0, 256, (d.V, d.H // 2), generator=g, device=dev, dtype=torch.uint8)
        scales = ((torch.rand((d.V, d.H // 128), generator=g, device=dev) * 0.4 + 0.8) * (d.lm_std / 2.5)).to(bf)
        lm = bdd.pack_lm_head_int4(codes, scales)
        wdt = bdd.BDD_INT4
    else:
        layer = {"w_router": rnd((d.E, d.H), d.w_std), "router_bias": bias,
                 "w_gate_up": rnd((d.E, 2 * d.I, d.H), d.w_std), "w_down": rnd((d.E, d.H, d.I), d.w_std),
                 "ws_gate_up": rnd((2 * d.I_s, d.H), d.w_std), "ws_down": rnd((d.H, d.I_s), d.w_std)}
        lm = bdd.pack_lm_head(rnd((d.V, d.H), d.lm_std))
        wdt = bdd.BDD_BF16
    plan = bdd.RoundPlan(bdd.MoEDims(d.T, d.H, d.E, d.K, d.I, d.I_s, wdt), [layer], lm, top_p, 0.95)
    x = torch.randn((d.T, d.H), generator=g, device=dev)
    tok = torch.full((d.T,), bdd.MASK, dtype=torch.int32, device=dev)
    conf = torch.empty(d.T, dtype=torch.float32, device=dev)
    choice = torch.empty(d.T, dtype=torch.int32, device=dev)
    ri = torch.empty(4, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        plan(x, tok, conf, choice, ri, None, nd)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run_rounds": 3, "mode": mode, "distinct_experts": int(nd.item())}), flush=True)


COUNTERS = os.path.join(ROOT, "profiles", "lmhead_clover_v248320_hbm_counters.md")
KERNEL_SOURCES = {"lmhead": ["lmhead.hip", "common.hpp", "kernels.hpp"]}


def lmhead_int4(args, d, dev, launches=200, copies=3):
    """The LM head with 4-bit weights (two codes per byte, code n standing for
    n - 8, one bf16 scale per row and 128 columns) + commit, on the Clover
    LM-head shape: average per-launch time from HIP events on the launch
    stream, against its algorithmic bytes (codes + scales + the block).  The
    packed weight (262 MB) fits in the 256 MiB memory-side cache, so the timed
    launches rotate over `copies` packed copies (each launch reads a weight the
    previous ones did not); the time over one copy is reported beside it."""
    import torch
    import block_diffusion_decode_amd as bdd
    import workloads as W

    codes, scales = W.lm_head_int4(args.seed, d, device=dev)
    lms = [bdd.pack_lm_head_int4(codes, scales) for _ in range(copies)]
    lm4 = lms[0]
    del codes, scales
    h = W.counter_normal(W.key_of(args.seed, "int4_h"), d.T * d.H, 1.0).to(torch.bfloat16)
    h = h.reshape(d.T, d.H).to(dev)
    ws = torch.empty(bdd.lmhead_workspace_bytes(d.T, d.H, d.V), dtype=torch.uint8, device=dev)
    tok = torch.full((d.T,), bdd.MASK, dtype=torch.int32, device=dev)
    conf = torch.empty(d.T, dtype=torch.float32, device=dev)
    choice = torch.empty(d.T, dtype=torch.int32, device=dev)
    ri = torch.empty(4, dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        tok.fill_(bdd.MASK)
        bdd.lmhead_confidence_commit(h, lm4, tok, ws=ws, conf=conf, choice=choice, round_info=ri)
    torch.cuda.synchronize()

    def timed(rotate):
        bdd.timing_enable(True, None)
        for i in range(launches):
            tok.fill_(bdd.MASK)
            bdd.lmhead_confidence_commit(h, lms[i % len(lms)] if rotate else lm4, tok, ws=ws, conf=conf,
                                         choice=choice, round_info=ri)
        torch.cuda.synchronize()
        t = bdd.timing_read()
        bdd.timing_enable(False)
        return t

    t = timed(True)
    t1 = timed(False)
    us = 1e3 * t["lmhead"][0] / t["lmhead"][1]
    us1 = 1e3 * t1["lmhead"][0] / t1["lmhead"][1]
    nbytes = d.V * d.H // 2 + d.V * (d.H // 128) * 2 + d.T * d.H * 2
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"LM head {d.V} x {d.H} with 4-bit weights (bf16 scale per 128 columns), block {d.T}, "
                        "+ LowConfidence commit (threshold 0.95)",
            "lmhead_us": round(us, 2), "commit_us": round(1e3 * t["commit"][0] / t["commit"][1], 2),
            "launches_timed": int(t["lmhead"][1]), "weight_copies_rotated": len(lms),
            "lmhead_us_one_copy": round(us1, 2), "algorithmic_bytes": nbytes, "achieved_gbps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def kernel_sha(kernel):
    """sha256 over the sources that define `kernel` (None if unknown)."""
    files = KERNEL_SOURCES.get(kernel)
    if not files:
        return None
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_diffusion_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the kernel's current sources; else (None, reason)."""
    sha = kernel_sha(kernel)
    if sha is None or not os.path.exists(COUNTERS):
        return None, "no counter summary for this kernel"
    text = open(COUNTERS).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_k = re.search(r"kernel:\s*(\w+)", text)
    if not (m_sha and m_b and m_k) or m_k.group(1) != kernel:
        return None, "counter summary unreadable"
    if m_sha.group(1) != sha:
        return None, "kernel changed since the counters were taken"
    return float(m_b.group(1)), os.path.relpath(COUNTERS, ROOT)


def cpu_baseline(args, d, x, layer, w_lm, info, budget_s):
    """The CPU oracle (float64 NumPy) on the same round, inputs already in host
    memory as float64; rounds run until the time budget is spent, with BLAS on
    every host thread, then a shorter sample on one thread."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count()
    log("[bench] preparing float64 host copies for the CPU oracle")
    L = {"w_router": layer["w_router"].double().cpu().numpy(),
         "router_bias": layer["router_bias"].double().cpu().numpy(),
         "ws_gate_up": layer["ws_gate_up"].double().cpu().numpy(),
         "ws_down": layer["ws_down"].double().cpu().numpy()}
    gu, dn = layer["w_gate_up"], layer["w_down"]
    L["experts"] = {e: (gu[e].double().cpu().numpy(), dn[e].double().cpu().numpy()) for e in range(d.E)}
    wl = w_lm.double().cpu().numpy()
    xs = x.double().cpu().numpy()

    def sample(seconds):
        tok = np.full(d.T, O.MASK)
        times = []
        t_end = time.perf_counter() + seconds
        r = 0
        while time.perf_counter() < t_end or r == 0:
            t0 = time.perf_counter()
            hh, _ = O.moe_stack(xs[r % xs.shape[0]], [L], d.K, 1.0)
            c, ch, _ = O.lm_head_confidence(hh, wl)
            tok, *_ = O.commit(tok, c, ch, 0.95)
            times.append(time.perf_counter() - t0)
            r += 1
        return 1e6 * float(np.median(times)), len(times)

    us, n = sample(budget_s)
    log(f"[bench] cpu oracle: {n} rounds, median {us / 1e3:.1f} ms/round on {threads} threads")
    out = {"value": round(us, 1), "unit": "us/round", "cores": threads, "kind": "oracle",
           "host_cpus": os.cpu_count(),
           "sample": f"{n} full rounds of the same workload (float64 NumPy oracle, median), BLAS on {threads} "
                     f"threads, inputs prepared as float64 host arrays before timing"}
    if threadpool_limits is not None:
        with threadpool_limits(1):
            us1, n1 = sample(budget_s / 3)
        log(f"[bench] cpu oracle, one thread: {n1} rounds, median {us1 / 1e3:.1f} ms/round")
        out["single_thread"] = {"value": round(us1, 1), "unit": "us/round", "cores": 1, "rounds": n1}
    return out


if __name__ == "__main__":
    main()
