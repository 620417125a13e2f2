"""Benchmark of the TP1 decode projection on one MI355X.

Default run (prints ONE JSON line):

* Headline: the multi-layer decode stream, the largest single-GPU workload
  of the five: 8 layers, each a distinct input-projection weight W_in
  [14560, 7168] then a distinct o_proj weight W_o [7168, 12288] (3.08 GB of
  weights in all, far more than the 256 MB MALL), B = 64, the o_proj input
  being columns 0..12287 of the in-projection output, x0 [64, 7168].  All
  inputs are the seeded recipe of `workloads.config_tensors` (seed 4), the
  same tensors the GPU parity tests check.  One step = one pass of the
  chain (16 projection calls on one stream, enqueued by one native call).
    value     = algorithmic bytes of a step (W + x + y of each call, once)
                / host-timed seconds per step, GB/s
    roofline  = the step's dominant kernel (the projection family with the
                most time per step), its algorithmic bytes per launch over
                its average launch time, both measured live here with HIP
                events on the launch stream, against the 8 TB/s HBM peak
    kernels   = both projections' average launch time and rate
    layer_us  = each layer's time (its two calls) in the chain, median over
                passes with an event between layers
* per_config: every batch point of the other four workloads (DSA B=1, the
  o_proj sweep, the KDA sweep, the DSA sweep to B=256), each call on a
  distinct weight copy from a rotation of >= 1 GB (cold: no call finds its
  weight in the MALL): us per call back to back (one pair of events around
  the calls) and by per-call event pairs (median, p10, p90), GB/s, % of 8 TB/s and %
  of the box's sustained read rate (the 2 GB read of read_ceiling);
  TFLOP/s and % of the 2.5 PFLOP/s BF16 MFMA peak for B >= 64.
* read_ceiling: the library's streaming-read probe over the chain's weights
  back to back and over a 2 GB buffer (the box's plain read rates).
* prefetch_overlap: the chain with a 10, 20 or 40 us memory-free stand-in for
  the attention core between each layer's projections, without and with the
  prefetch of the head (or all) of that layer's o_proj weight while the core
  runs: on a second stream (fork/join), or inside the stand-in's own launch.
* moe_front: the MoE layer's split-K front, one projection over a packed
  [part 0 | part 1] weight (proj_pack_rows) against the two parts as separate
  projections, cold, at K = 7168 and B = 1..64; the pages print neither
  part's size, so the parts sweep 2048+1024, 4096+2048 and 8192+4096 rows.
* cpu_baseline: the CPU oracle (FP64 sums) on the same chain, on all host
  cores, over a bounded number of layers; its CPU model; a one-thread
  figure for the DSA B=1 workload; and one call of each single-projection
  workload at its largest batch.

`--ring-probe` times only the projection kernel's LDS-ring loads without its
arithmetic (proj_ring_probe): x alone, the weight alone, both, and variants of
piece width, barrier and bytes in flight.

`--report PATH` also writes every point's hot figure (one weight repeated,
cache-assisted) and the graph-replayed chain to PATH as JSON.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call + achieved HBM GB/s (% of peak), TP1 BF16 decode projections, B=1..64"
SWEEPS = ("dsa_b1", "oproj_sweep", "kda_sweep", "dsa_sweep")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="after the warmup steps, keep stepping (untimed) until this much "
                         "time has passed, so the timed steps do not run at ramping clocks")
    ap.add_argument("--report", default=None,
                    help="also write hot figures and the graph-replayed chain here")
    ap.add_argument("--configs", default=None,
                    help="comma-separated workloads for per_config (default: all four); "
                         "'none' skips them")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the multi-layer stream (e.g. under a profiler)")
    ap.add_argument("--sweeps-only", action="store_true",
                    help="time only the per_config workloads and print them as one JSON "
                         "line (e.g. under a profiler, without the stream's dispatches)")
    ap.add_argument("--front-only", action="store_true",
                    help="time only the MoE front study and print it as one JSON line")
    ap.add_argument("--front-reps", type=int, default=40,
                    help="timed rounds per MoE front point (fewer under a profiler)")
    ap.add_argument("--front-sizes", default=None,
                    help="comma-separated indices of the MoE front sizes to time (default: all)")
    ap.add_argument("--front-no-separate", action="store_true",
                    help="skip the separate-launch comparison (a profile then holds only "
                         "front launches)")
    ap.add_argument("--ring-probe", action="store_true",
                    help="time only the LDS-ring load probe (the projection kernel's loads "
                         "without its arithmetic) and print it as one JSON line")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time of the bounded oracle sample (whole layers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times, the known-size "
                         "reference that scales FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def copy_calibration(torch):
    """A plain device-to-device copy of 256 MiB: reads and writes exactly
    268435456 bytes, so profiler byte counters can be scaled by it."""
    n = 256 * 1024 * 1024 // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    _say("copy calibration: 5 x 268435456-byte device copies done")


def measured_traffic(kernel: str, B: int, N: int):
    """HBM bytes per launch of `kernel` (a [B, N] output) from the committed
    counter summary (profiles/traffic.json), or None when it was taken from
    another version of the kernel source or never taken.  A split-K call is
    the main kernel plus the reduction pass, whose entry is keyed by its grid
    (it serves every shape under one name)."""
    from tp1_skinny_bf16_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != profile_summary.source_hash():
        return None
    total = 0
    for part in kernel.split("+"):
        key = part
        if part.startswith("splitk_reduce4<"):
            key = f"{part}@{-(-B * N // 4 // 256) * 256}"
        elif part.startswith("splitk_reduce<"):
            key = f"{part}@{-(-B * N // 256) * 256}"
        entry = data.get("kernels", {}).get(key)
        if not entry:
            return None
        total += entry["traffic"]
    return int(total)


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def headline(args, torch, tp, wl, timing):
    """The multi-layer stream on the seed-4 tensors."""
    cfg = wl.BY_NAME["multilayer"]
    t = wl.config_tensors(cfg)
    dev = torch.device("cuda:0")
    B, L = cfg.bmax, cfg.layers
    w_in = [w.to(dev) for w in t["W_in"]]
    w_o = [w.to(dev) for w in t["W_o"]]
    x0 = t["x"].to(dev)
    pin = tp.Plan(wl.DSA_N, wl.DSA_K, [B])
    po = tp.Plan(wl.OPROJ_N, wl.OPROJ_K, [B])
    stack = tp.LayerStack(pin, po, w_in, w_o)
    y_in, y_o = stack.buffers(B)
    stream = torch.cuda.current_stream()

    def step():
        stack.run(x0, y_in, y_o)

    for _ in range(args.warmup):
        step()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.warm_seconds:
        for _ in range(5):
            step()
        torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
    b_in = wl.algorithmic_bytes(B, wl.DSA_N, wl.DSA_K)
    b_o = wl.algorithmic_bytes(B, wl.OPROJ_N, wl.OPROJ_K)
    step_bytes = L * (b_in + b_o)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # Each projection family alone, in the chain's own launch configuration:
    # the 8 layers' calls back to back on the launch stream (distinct weights,
    # each call's own chain input), one pair of events around args.steps
    # rounds of them.
    sh = stream.cuda_stream
    xin = [x0] + [y_o[l - 1] for l in range(1, L)]

    def run_in(l):
        rc = pin.run_ptr(B, xin[l].data_ptr(), wl.DSA_K, w_in[l].data_ptr(),
                         y_in[l].data_ptr(), sh)
        if rc != 0:
            raise tp.ProjError(rc, "in-projection")

    def run_o(l):
        rc = po.run_ptr(B, y_in[l].data_ptr(), wl.DSA_N, w_o[l].data_ptr(),
                        y_o[l].data_ptr(), sh)
        if rc != 0:
            raise tp.ProjError(rc, "o_proj")

    fam = {}
    for name, fn, nbytes, plan, N, K in (("in_proj", run_in, b_in, pin, wl.DSA_N, wl.DSA_K),
                                          ("o_proj", run_o, b_o, po, wl.OPROJ_N, wl.OPROJ_K)):
        for l in range(L):
            fn(l)
        torch.cuda.synchronize()
        a, b = _events(torch, 2)
        a.record(stream)
        for _ in range(args.steps):
            for l in range(L):
                fn(l)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (args.steps * L)
        fam[name] = {"kernel": plan.kernel_name(B), "shape": f"{N}x{K}", "B": B,
                     "us_per_launch": round(us, 2), "bytes_per_launch": nbytes,
                     "GBps": round(timing.gbs(nbytes, us), 1),
                     "pct_peak": round(100 * timing.gbs(nbytes, us) / timing.HBM_PEAK_GBS, 1),
                     "TFLOPs": round(2.0 * B * N * K / (us * 1e-6) / 1e12, 1)}
    # Each layer of the chain: the step's calls in order, an event after each
    # layer, median over `steps` passes (a separate pass: the events between
    # layers are not in the timed region above).
    per_layer = [[] for _ in range(L)]
    for _ in range(max(3, args.steps // 5)):
        ev = _events(torch, L + 1)
        ev[0].record(stream)
        for l in range(L):
            run_in(l)
            run_o(l)
            ev[l + 1].record(stream)
        torch.cuda.synchronize()
        for l in range(L):
            per_layer[l].append(ev[l].elapsed_time(ev[l + 1]) * 1e3)
    layer_us = [round(sorted(v)[len(v) // 2], 2) for v in per_layer]
    # restore the chain's outputs (the per-family passes rewrote them in place
    # with the same values, in the same order, so this is only for clarity)
    step()
    torch.cuda.synchronize()
    dom_name = max(fam, key=lambda k: fam[k]["us_per_launch"])
    dom = fam[dom_name]
    achieved = timing.gbs(dom["bytes_per_launch"], dom["us_per_launch"])
    roof = {"bound": "hbm", "kernel": dom["kernel"], "role": dom_name,
            "achieved": round(achieved, 1), "peak": timing.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / timing.HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom["kernel"], B,
                                        wl.DSA_N if dom_name == "in_proj" else wl.OPROJ_N),
            "avg_launch_us": dom["us_per_launch"],
            "bytes_per_launch": dom["bytes_per_launch"]}

    # read ceilings: the chain's own weights read back to back by the plain
    # streaming-read probe (one launch per weight), and a 2 GB buffer
    sink = torch.empty(65536, dtype=torch.float32, device=dev)
    rl = timing.time_calls([(lambda W=W: tp.read_probe(W, sink, 4)) for W in w_in],
                           warmup=2, reps=4 * L, warm_seconds=0.05)
    big = torch.ones(1024 ** 3, dtype=torch.bfloat16, device=dev)
    rs = timing.time_calls([lambda: tp.read_probe(big, sink, 4)], warmup=2, reps=10,
                           warm_seconds=0.05)
    wbytes = wl.DSA_N * wl.DSA_K * 2
    per_launch = timing.gbs(wbytes, rl["us_mean_b2b"])
    ceiling = {"in_proj_weight_read_us": round(rl["us_mean_b2b"], 2),
               "in_proj_weight_read_GBps": round(per_launch, 1),
               "sustained_2GB_GBps": round(timing.gbs(big.numel() * 2, rs["us_median"]), 1)}
    del big
    overlap = overlap_study(torch, wl, timing, stack, x0, y_in, y_o, reps=max(5, args.steps // 2))
    graph = None
    if args.report:
        graph = timing.time_graph([step], replays=10)
    return {"cfg": cfg, "t": t, "value": value, "ms": ms_per_step, "layer_us": layer_us,
            "gpu_ms": gpu_ms_per_step, "step_bytes": step_bytes, "families": fam,
            "roofline": roof, "read_ceiling": ceiling, "graph_us": graph, "overlap": overlap,
            "stack": stack, "tensors": (w_in, w_o, x0, y_in, y_o)}


def overlap_study(torch, wl, timing, stack, x0, y_in, y_o, reps):
    """The chain with a memory-free stand-in for the attention core between
    each layer's projections, without and with the prefetch of the head of
    that layer's o_proj weight on a second stream during the core (the
    runtime page's L2 weight prefetch, forked and joined around the core as
    the hybrid page's NoPrefetch interface does).  us per step."""
    side = torch.cuda.Stream()               # default priority
    stream = torch.cuda.current_stream()
    wo_bytes = wl.OPROJ_N * wl.OPROJ_K * 2

    def timed(core_us, pf, in_core=False):
        kw = dict(core_us=core_us, prefetch_bytes=pf,
                  side_stream=side if pf and not in_core else None, prefetch_in_core=in_core)
        for _ in range(3):
            stack.run_overlap(x0, y_in, y_o, **kw)
        torch.cuda.synchronize()
        a, b = _events(torch, 2)
        a.record(stream)
        for _ in range(reps):
            stack.run_overlap(x0, y_in, y_o, **kw)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    # the most a prefetch can give: o_proj right after its whole weight was
    # read into the caches, against o_proj cold (the chain's own order)
    B = x0.shape[0]
    pin, po = stack.in_plan, stack.out_plan
    sh = stream.cuda_stream

    def o_proj(l):
        rc = po.run_ptr(B, y_in[l].data_ptr(), wl.DSA_N, stack.w_o[l].data_ptr(),
                        y_o[l].data_ptr(), sh)
        assert rc == 0

    def in_proj(l):
        x = x0 if l == 0 else y_o[l - 1]
        rc = pin.run_ptr(B, x.data_ptr(), wl.DSA_K, stack.w_in[l].data_ptr(),
                         y_in[l].data_ptr(), sh)
        assert rc == 0

    cold, warm, pf_us = [], [], []
    from tp1_skinny_bf16_amd import prefetch
    for rep in range(reps):
        for l in range(stack.layers):
            e = _events(torch, 6)
            in_proj(l)
            e[0].record(stream)
            o_proj(l)                                  # cold: straight after in-proj
            e[1].record(stream)
            in_proj(l)                                 # evict with the in-proj weight again
            e[2].record(stream)
            prefetch(stack.w_o[l], wo_bytes)           # whole o_proj weight
            e[3].record(stream)
            o_proj(l)
            e[4].record(stream)
            torch.cuda.synchronize()
            if rep > 0:
                cold.append(e[0].elapsed_time(e[1]) * 1e3)
                pf_us.append(e[2].elapsed_time(e[3]) * 1e3)
                warm.append(e[3].elapsed_time(e[4]) * 1e3)
    out = {"layers": stack.layers, "o_proj_weight_bytes": wo_bytes,
           "o_proj_us_cold": round(sum(cold) / len(cold), 2),
           "o_proj_us_after_full_prefetch": round(sum(warm) / len(warm), 2),
           "full_prefetch_us": round(sum(pf_us) / len(pf_us), 2),
           "full_prefetch_GBps": round(timing.gbs(wo_bytes, sum(pf_us) / len(pf_us)), 1),
           "points": []}
    # Per core duration: the chain without prefetch, then with the head the
    # core's duration could fetch at ~4.5 TB/s (the cached-load rate) and with
    # the whole weight, each prefetched on a second stream (fork/join) and
    # inside the stand-in's own launch (no second stream).  us per step.
    for core_us in (10.0, 20.0, 40.0):
        base = timed(core_us, 0)
        row = {"core_us": core_us, "chain_us_no_prefetch": round(base, 1),
               "side_stream": {}, "in_core_launch": {}}
        for pf in sorted({min(wo_bytes, int(core_us * 4.5e6)) // 16 * 16, wo_bytes}):
            row["side_stream"][str(pf)] = round(timed(core_us, pf), 1)
            row["in_core_launch"][str(pf)] = round(timed(core_us, pf, in_core=True), 1)
        out["points"].append(row)
    _say(f"prefetch beside the core stand-in: {out}")
    return out


def per_config(args, torch, tp, wl, timing, report, ceiling_gbps=None):
    """Every batch point of the four single-projection workloads, cold; with
    the box's sustained read rate (GB/s) known, also each point's share of it."""
    dev = torch.device("cuda:0")
    names = SWEEPS if args.configs is None else \
        tuple(n for n in args.configs.split(",") if n and n != "none")
    unknown = set(names) - set(SWEEPS)
    if unknown:
        raise SystemExit(f"unknown workloads: {sorted(unknown)}")
    out = {}
    for name in names:
        cfg = wl.BY_NAME[name]
        t = wl.config_tensors(cfg)
        W0 = t["W"].to(dev)
        x = t["x"].to(dev)
        copies = timing.rotation_copies(W0)
        plan = tp.Plan(cfg.N, cfg.K, cfg.batches)
        pts = {}
        for B in cfg.batches:
            y = torch.empty((B, cfg.N), dtype=torch.bfloat16, device=dev)
            xb = x[:B]
            calls = [(lambda W=W: plan.run(xb, W, y)) for W in copies]
            cold = timing.time_calls(calls, warmup=3, reps=60)
            nbytes = wl.algorithmic_bytes(B, cfg.N, cfg.K)
            b2b = cold["us_mean_b2b"]
            p = {"us_b2b": round(b2b, 2), "us_median": round(cold["us_median"], 2),
                 "us_p10": round(cold["us_p10"], 2), "us_p90": round(cold["us_p90"], 2),
                 "GBps_b2b": round(timing.gbs(nbytes, b2b), 1),
                 "pct_peak_b2b": round(100 * timing.gbs(nbytes, b2b) / timing.HBM_PEAK_GBS, 1),
                 "pct_peak_median": round(100 * timing.gbs(nbytes, cold["us_median"])
                                          / timing.HBM_PEAK_GBS, 1),
                 "kernel": plan.kernel_name(B)}
            if ceiling_gbps:
                p["pct_read_ceiling_b2b"] = round(100 * timing.gbs(nbytes, b2b) / ceiling_gbps, 1)
            if B >= 64:
                tf = 2.0 * B * cfg.N * cfg.K / (b2b * 1e-6) / 1e12
                p["TFLOPs_b2b"] = round(tf, 1)
                p["pct_mfma_peak_b2b"] = round(100 * tf / timing.MFMA_BF16_PEAK_TFLOPS, 1)
            if report is not None:
                hot = timing.time_calls([lambda: plan.run(xb, W0, y)], warmup=3, reps=30)
                p["hot_us_median"] = round(hot["us_median"], 2)
            pts[str(B)] = p
            _say(f"{name:12s} B={B:3d} b2b {p['us_b2b']:7.2f} us {p['GBps_b2b']:7.1f} GB/s "
                 f"({p['pct_peak_b2b']:4.1f}%)  per call {p['us_median']:7.2f} us  "
                 f"{p['kernel']}")
        out[name] = {"N": cfg.N, "K": cfg.K, "seed": cfg.seed, "weight_copies": len(copies),
                     "points": pts}
        del copies, W0, x, t, plan
        torch.cuda.empty_cache()
    return out


FRONT_PARTS = ((2048, 1024), (4096, 2048), (8192, 4096))
FRONT_BATCHES = (1, 4, 16, 64)


def moe_front(args, torch, tp, wl, timing):
    """The MoE front: one projection over the packed [part 0 | part 1] weight
    against the two parts as separate projections, cold, at K = 7168.  The
    pages print neither part's size, so the rows sweep (2/3 and 1/3 of N)."""
    dev = torch.device("cuda:0")
    K = wl.DSA_K
    sizes = range(len(FRONT_PARTS)) if args.front_sizes is None else \
        [int(v) for v in args.front_sizes.split(",")]
    out = {"K": K, "parts_rows": [list(FRONT_PARTS[i]) for i in sizes], "points": []}
    for i in sizes:
        n0, n1 = FRONT_PARTS[i]
        x, W0 = wl.random_case(max(FRONT_BATCHES), n0, K, seed=40 + i)
        _, W1 = wl.random_case(1, n1, K, seed=50 + i)
        x = x.to(dev)
        packed = tp.pack_rows([W0.to(dev), W1.to(dev)])
        copies = timing.rotation_copies(packed)
        N = n0 + n1
        front = tp.Plan(N, K, list(FRONT_BATCHES))
        p0, p1 = tp.Plan(n0, K, list(FRONT_BATCHES)), tp.Plan(n1, K, list(FRONT_BATCHES))
        for B in FRONT_BATCHES:
            xb = x[:B]
            y = torch.empty((B, N), dtype=torch.bfloat16, device=dev)
            y0 = torch.empty((B, n0), dtype=torch.bfloat16, device=dev)
            y1 = torch.empty((B, n1), dtype=torch.bfloat16, device=dev)
            one = timing.time_calls([(lambda W=W: front.run(xb, W, y)) for W in copies],
                                    warmup=3, reps=args.front_reps)

            def both(W):
                p0.run(xb, W[:n0], y0)
                p1.run(xb, W[n0:], y1)
            two = None if args.front_no_separate else timing.time_calls(
                [(lambda W=W: both(W)) for W in copies], warmup=3, reps=args.front_reps)
            nbytes = wl.algorithmic_bytes(B, N, K)
            row = {"rows": [n0, n1], "N": N, "K": K, "B": B,
                   "front_us_b2b": round(one["us_mean_b2b"], 2),
                   "separate_us_b2b": round(two["us_mean_b2b"], 2) if two else None,
                   "front_GBps_b2b": round(timing.gbs(nbytes, one["us_mean_b2b"]), 1),
                   "front_pct_peak_b2b": round(100 * timing.gbs(nbytes, one["us_mean_b2b"])
                                               / timing.HBM_PEAK_GBS, 1),
                   "kernel": front.kernel_name(B)}
            out["points"].append(row)
            _say(f"moe front {n0}+{n1} B={B:2d}: one launch {row['front_us_b2b']:6.2f} us "
                 f"({row['front_pct_peak_b2b']:4.1f}%), two launches {row['separate_us_b2b']} us")
        for pl in (front, p0, p1):
            pl.close()
        del copies, packed
        torch.cuda.empty_cache()
    return out


# (label, stage rows, piece bytes, stages, barrier, what, shared weight)
RING_CASES = (
    ("x only", 64, 256, 5, 1, 1, 0),
    ("weight only (a private block per workgroup: HBM)", 64, 256, 5, 1, 2, 0),
    ("weight only (one block for all: L2 / MALL)", 64, 256, 5, 1, 2, 1),
    ("x + private weight", 128, 256, 3, 1, 3, 0),
    ("x + shared weight", 128, 256, 3, 1, 3, 1),
    ("x only, no barrier", 64, 256, 5, 0, 1, 0),
    ("x only, 512-byte pieces", 64, 512, 3, 1, 1, 0),
    ("x only, 512-byte pieces, no barrier", 64, 512, 3, 0, 1, 0),
    ("x only, 1 KB pieces", 64, 1024, 2, 1, 1, 0),
    ("x only, 1 KB pieces, no barrier", 64, 1024, 2, 0, 1, 0),
    ("x only, twice the bytes in flight", 64, 256, 9, 1, 1, 0),
    ("x + private weight, twice the bytes in flight", 128, 256, 5, 1, 3, 0),
    ("x only, 128-byte pieces", 64, 128, 9, 1, 1, 0),
    ("weight only (private), 128-byte pieces", 64, 128, 9, 1, 2, 0),
    ("x + private weight, 128-byte pieces", 128, 128, 9, 1, 3, 0),
)


def ring_probe_study(torch, tp, timing):
    """The pipelined kernel's LDS-ring loads alone (proj_ring_probe) over 256
    workgroups, one per compute unit, each reading 917,504 bytes per 64
    stage rows (64 rows x 7168 BF16): x, shared by every workgroup, and the
    weight, a private block per workgroup (two copies alternated, 470 MB, so
    it comes from HBM) or one block for all."""
    dev = torch.device("cuda:0")
    K, grid = 7168, 256
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    x = (torch.randn((64, K), generator=g, device=dev)).to(torch.bfloat16)
    ws = [(torch.randn((grid * 64, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
          for _ in range(2)]
    sink = torch.empty(grid * 8, dtype=torch.float32, device=dev)
    out = []
    for label, rows, piece, depth, barrier, what, shared in RING_CASES:
        calls = [(lambda w=w: tp.ring_probe(x, w, rows=rows, piece=piece, depth=depth,
                                            barrier=bool(barrier), what=what,
                                            shared_w=bool(shared), grid=grid, sink=sink))
                 for w in ws]
        r = timing.time_calls(calls, warmup=3, reps=40, warm_seconds=0.05)
        per_cu = rows * K * 2
        row = {"case": label, "rows": rows, "piece": piece, "stages": depth,
               "inflight_KB": (depth - 1) * rows * piece // 1024, "barrier": bool(barrier),
               "us_b2b": round(r["us_mean_b2b"], 2),
               "GBps_per_CU": round(per_cu / r["us_mean_b2b"] / 1e3, 1)}
        out.append(row)
        _say(f"ring probe {label:48s} {row['us_b2b']:6.2f} us  {row['GBps_per_CU']:5.1f} GB/s per CU")
    return {"K": K, "workgroups": grid, "bytes_per_64_rows": 64 * K * 2, "cases": out}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, h, wl):
    """The oracle on the multi-layer stream, layer by layer, chained on its
    own outputs, until cpu_seconds have passed; one thread on DSA B=1; and one
    call of every single-projection workload at its largest batch."""
    import oracle
    cfg, t = h["cfg"], h["t"]
    threads = oracle.default_threads()
    xb = wl.bits(t["x"])
    oracle.proj(xb[:1], wl.bits(t["W_in"][0])[:64], threads=threads)   # load the library
    b_in = wl.algorithmic_bytes(cfg.bmax, wl.DSA_N, wl.DSA_K)
    b_o = wl.algorithmic_bytes(cfg.bmax, wl.OPROJ_N, wl.OPROJ_K)
    done, nbytes, x = 0, 0, xb
    t0 = time.perf_counter()
    while True:
        l = done % cfg.layers
        if l == 0:
            x = xb
        yi = oracle.proj(x, wl.bits(t["W_in"][l]), threads=threads)
        yo = oracle.proj(yi[:, :wl.OPROJ_K], wl.bits(t["W_o"][l]), threads=threads)
        x = yo
        done += 1
        nbytes += b_in + b_o
        if time.perf_counter() - t0 >= args.cpu_seconds or done >= 4 * cfg.layers:
            break
    el = time.perf_counter() - t0
    # one thread, DSA B=1 (the first workload)
    c1 = wl.config_tensors(wl.BY_NAME["dsa_b1"])
    x1, w1 = wl.bits(c1["x"]), wl.bits(c1["W"])
    t1 = time.perf_counter()
    oracle.proj(x1, w1, threads=1)
    e1 = time.perf_counter() - t1
    n1 = wl.algorithmic_bytes(1, wl.DSA_N, wl.DSA_K)
    # every single-projection workload: one call at its largest batch, all threads
    per_cfg = {}
    for name in SWEEPS:
        c = wl.BY_NAME[name]
        ct = wl.config_tensors(c)
        xb_c, wb_c = wl.bits(ct["x"]), wl.bits(ct["W"])
        B = c.bmax
        tc = time.perf_counter()
        oracle.proj(xb_c[:B], wb_c, threads=threads)
        ec = time.perf_counter() - tc
        per_cfg[name] = {"B": B, "ms_per_call": round(ec * 1e3, 1),
                         "GBps": round(wl.algorithmic_bytes(B, c.N, c.K) / ec / 1e9, 3)}
        del ct, xb_c, wb_c
    return {"value": round(nbytes / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{done} layers (in-projection then o_proj, B=64) of the 8-layer "
                      f"stream on the seed-4 tensors, chained on the oracle's own outputs, "
                      f"{el:.1f} s, FP64 sums",
            "ms_per_layer": round(el * 1e3 / done, 1),
            "ms_per_step_extrapolated": round(el * 1e3 / done * cfg.layers, 1),
            "t1_dsa_b1": {"threads": 1, "ms_per_call": round(e1 * 1e3, 1),
                          "GBps": round(n1 / e1 / 1e9, 3)},
            "per_config": per_cfg}


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "the projection is measured on one GPU: it runs one "
                          "DEP rank's share, and this library neither shards nor "
                          "communicates across GPUs; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import tp1_skinny_bf16_amd as tp
    import workloads as wl
    from tp1_skinny_bf16_amd import timing

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.ring_probe:
        print(json.dumps({"ring_probe": ring_probe_study(torch, tp, timing)}), flush=True)
        return
    if args.front_only:
        front = moe_front(args, torch, tp, wl, timing)
        if args.copy_calibration:
            copy_calibration(torch)
        print(json.dumps({"moe_front": front}), flush=True)
        return
    if args.sweeps_only:
        pc = per_config(args, torch, tp, wl, timing, None)
        if args.copy_calibration:
            copy_calibration(torch)
        print(json.dumps({"per_config": pc}), flush=True)
        return
    _say("timing the 8-layer stream (seed-4 tensors)")
    h = headline(args, torch, tp, wl, timing)
    _say(f"8-layer stream: {h['ms'] * 1e3:.1f} us/step, {h['value']:.1f} GB/s; "
         f"{h['families']}")
    report = {} if args.report else None
    pc = None
    if not args.headline_only and args.configs != "none":
        pc = per_config(args, torch, tp, wl, timing, report,
                        ceiling_gbps=h["read_ceiling"]["sustained_2GB_GBps"])
    front = None
    if not args.headline_only and args.configs != "none":
        front = moe_front(args, torch, tp, wl, timing)
    cpu = None
    if not args.no_cpu and not args.headline_only:
        _say("timing the CPU oracle")
        cpu = cpu_baseline(args, h, wl)
    if args.copy_calibration:
        copy_calibration(torch)
    cfg = h["cfg"]
    line = {
        "metric": METRIC,
        "value": round(h["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_seconds": args.warm_seconds,
        "ms_per_step": round(h["ms"], 4),
        "gpu_ms_per_step": round(h["gpu_ms"], 4),
        "us_per_call": round(h["ms"] * 1e3 / (2 * cfg.layers), 2),
        "pct_peak": round(100 * h["value"] / timing.HBM_PEAK_GBS, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "multi-layer decode stream: 8 layers x (W_in 14560x7168 then "
                               "W_o 7168x12288, distinct BF16 ~N(0,0.02) weights, 3.08 GB), "
                               "B=64, o_proj input = columns 0..12287 of the in-projection "
                               "output, x0[64,7168] ~N(0,1), seed 4; one step = the chain",
                   "layers": cfg.layers, "B": cfg.bmax, "step_bytes": h["step_bytes"],
                   "calls_per_step": 2 * cfg.layers},
        "kernels": h["families"],
        "layer_us": h["layer_us"],
        "roofline": h["roofline"],
        "read_ceiling": h["read_ceiling"],
        "prefetch_overlap": h["overlap"],
        "per_config": pc,
        "moe_front": front,
        "cpu_baseline": cpu,
    }
    if args.report:
        report["headline"] = {k: line[k] for k in ("value", "ms_per_step", "kernels")}
        report["graph_replayed_chain_us"] = h["graph_us"]
        report["per_config"] = pc
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
