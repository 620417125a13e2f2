"""Benchmark of the TP1 decode projection on one MI355X.

Default run: the o_proj sweep workload (W 7168 x 12288 BF16, x[B, 12288],
B = 1, 2, 4, 8, 16, seed 1).  One step = one projection call per batch size,
each on its own weight copy from a rotation of distinct copies (>= 1 GB in
total, so no call finds its weight in the 256 MB MALL).  Inputs are resident
in HBM before timing starts.  Prints ONE JSON line:
  value        = algorithmic HBM bytes of a step / step time, GB/s
  roofline     = the dominant kernel's achieved GB/s against the 8 TB/s peak
  read_ceiling = a plain streaming read of the same weight copies, one launch
                 per copy, and of a 2 GB buffer, measured after the timed
                 region; the dominant kernel as a fraction of the former
  cpu_baseline = the CPU oracle timed on a bounded sample of the same step

`--report PATH` also times every point of every configuration (DSA B=1, the
o_proj, KDA and DSA sweeps, the 8-layer stream), the plain streaming-read
ceiling and the cache-assisted ("hot", one weight repeated) figures, and
writes them as JSON to PATH.
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

HEADLINE = "oproj_sweep"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="after the warmup steps, keep stepping (untimed) until this much "
                         "time has passed, so the timed steps do not run at ramping clocks")
    ap.add_argument("--report", default=None, help="write the all-config report here")
    ap.add_argument("--configs", default=None,
                    help="with --report: comma-separated configuration names to time "
                         "(default all, with the read ceiling and the multi-layer chain)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time of the bounded oracle sample (whole steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy 5 times, the known-size "
                         "reference that scales FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


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


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def headline(args, torch, tp, wl, timing):
    cfg = wl.BY_NAME[HEADLINE]
    t = wl.config_tensors(cfg)
    dev = torch.device("cuda:0")
    W0 = t["W"].to(dev)
    x = t["x"].to(dev)
    copies = timing.rotation_copies(W0)
    plan = tp.Plan(cfg.N, cfg.K, cfg.batches)
    outs = {B: torch.empty((B, cfg.N), dtype=torch.bfloat16, device=dev) for B in cfg.batches}
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    xs = {B: x[:B] for B in cfg.batches}
    nb = len(cfg.batches)
    ncopy = len(copies)

    def call(i, B):
        W = copies[i % ncopy]
        rc = plan.run_ptr(B, xs[B].data_ptr(), cfg.K, W.data_ptr(), outs[B].data_ptr(), sh)
        if rc != 0:
            raise tp.ProjError(rc, f"proj_run B={B}")

    def step(s):
        for j, B in enumerate(cfg.batches):
            call(s * nb + j, B)

    for s in range(args.warmup):
        step(s)
    # A fresh process starts at low clocks; a few ms of warm-up steps do not
    # raise them.  Keep stepping, untimed, until warm_seconds have passed.
    t_warm = time.perf_counter()
    s = args.warmup
    while time.perf_counter() - t_warm < args.warm_seconds:
        for _ in range(20):
            step(s)
            s += 1
        torch.cuda.synchronize()
    # Timed region: the K steps' calls, grouped by batch size (B-major) so that
    # each size's K calls run back to back between one pair of HIP events on
    # the launch stream; a step is still one call per batch size.
    ev = {B: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for B in cfg.batches}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j, B in enumerate(cfg.batches):
        ev[B][0].record(stream)
        for s in range(args.steps):
            call(s * nb + j, B)
        ev[B][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    step_bytes = sum(wl.algorithmic_bytes(B, cfg.N, cfg.K) for B in cfg.batches)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    per_b = {}
    for j, B in enumerate(cfg.batches):
        mean = ev[B][0].elapsed_time(ev[B][1]) * 1e3 / args.steps
        tac, _ = plan.tactic(B)
        per_b[B] = {"us_per_call": round(mean, 2),
                    "GBps": round(timing.gbs(wl.algorithmic_bytes(B, cfg.N, cfg.K), mean), 1),
                    "kernel": plan.kernel_name(B), "tactic": tac.as_dict()}
    # dominant kernel: the one with the largest share of the step's GPU time
    by_kernel = {}
    for B, r in per_b.items():
        k = by_kernel.setdefault(r["kernel"], {"us": 0.0, "bytes": 0, "calls": 0})
        k["us"] += r["us_per_call"]
        k["bytes"] += wl.algorithmic_bytes(B, cfg.N, cfg.K)
        k["calls"] += 1
    name, k = max(by_kernel.items(), key=lambda kv: kv[1]["us"])
    avg_us = k["us"] / k["calls"]
    bytes_per_launch = k["bytes"] / k["calls"]
    achieved = timing.gbs(bytes_per_launch, avg_us)
    roof = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1),
            "peak": timing.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / timing.HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(name),
            "avg_launch_us": round(avg_us, 2), "bytes_per_launch": int(bytes_per_launch)}
    # Read ceilings of the box, after the timed region: the library's
    # streaming-read probe (a plain 128-bit read-and-reduce, 4 waves per CU)
    # over the same rotated weight copies back to back, one launch per copy
    # (what a single-pass projection of this weight can reach per launch),
    # and over one 2 GB buffer (the sustained rate).
    sink = torch.empty(65536, dtype=torch.float32, device=dev)
    wbytes = cfg.N * cfg.K * 2
    rl = timing.time_calls([(lambda W=W: tp.read_probe(W, sink, 4)) for W in copies],
                           warmup=2, reps=4 * ncopy, warm_seconds=0.05)
    big = torch.ones(1024 ** 3, dtype=torch.bfloat16, device=dev)
    rs = timing.time_calls([lambda: tp.read_probe(big, sink, 4)], warmup=2, reps=10,
                           warm_seconds=0.05)
    per_launch = timing.gbs(wbytes, rl["us_mean_b2b"])
    ceiling = {"per_launch_GBps": round(per_launch, 1),
               "per_launch_us": round(rl["us_mean_b2b"], 2),
               "sustained_GBps": round(timing.gbs(big.numel() * 2, rs["us_median"]), 1),
               "dominant_kernel_frac_of_per_launch": round(achieved / per_launch, 4)}
    del big
    res = {"cfg": cfg, "t": t, "plan": plan, "value": value, "ms": ms_per_step,
           "per_b": per_b, "roofline": roof, "step_bytes": step_bytes,
           "copies": ncopy, "read_ceiling": ceiling}
    return res


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic.json), or None when it was taken from another version
    of the kernel source or never taken."""
    from tp1_skinny_bf16_amd import profile_summary
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != profile_summary.source_hash():
        return None
    total = 0
    for part in kernel.split("+"):   # a split-K call is the main kernel + splitk_reduce
        entry = data.get("kernels", {}).get(part)
        if not entry:
            return None
        total += entry["traffic"]
    return int(total)


def cpu_baseline(args, cfg, t, wl):
    import oracle
    xb = wl.bits(t["x"])
    wb = wl.bits(t["W"])
    threads = oracle.default_threads()
    oracle.proj(xb[:1], wb[:64], threads=threads)       # load / warm the library
    reps, t0 = 0, time.perf_counter()
    while True:
        for B in cfg.batches:
            oracle.proj(xb[:B], wb, threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= args.cpu_seconds or reps >= 1000:
            break
    el = time.perf_counter() - t0
    step_bytes = sum(wl.algorithmic_bytes(B, cfg.N, cfg.K) for B in cfg.batches)
    return {"value": round(step_bytes * reps / el / 1e9, 3), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{reps} full steps of the o_proj sweep (B=1,2,4,8,16 on one "
                      f"7168x12288 weight), {el:.1f} s, FP64 accumulation",
            "ms_per_step": round(el * 1e3 / reps, 1)}


def report(args, torch, tp, wl, timing):
    """Every configuration point, cold (rotated weights) and hot."""
    dev = torch.device("cuda:0")
    out = {"points": [], "device": torch.cuda.get_device_name(0)}
    names = set(args.configs.split(",")) if args.configs else None
    unknown = (names or set()) - set(wl.BY_NAME)
    if unknown:
        raise SystemExit(f"unknown configurations: {sorted(unknown)}")
    if names is None:
        # plain streaming-read ceiling over a 2 GB buffer
        buf = torch.empty(2 * 1024 ** 3 // 2, dtype=torch.bfloat16, device=dev)
        buf.fill_(1.0)
        sink = torch.empty(65536, dtype=torch.float32, device=dev)
        probe = {}
        for wpc in (4, 8, 16, 32):
            r = timing.time_calls([lambda: tp.read_probe(buf, sink, wpc)], warmup=3, reps=20)
            probe[wpc] = round(timing.gbs(buf.numel() * 2, r["us_median"]), 1)
        out["read_ceiling_GBps"] = probe
        _say(f"read ceiling (GB/s by waves/CU): {probe}")
        del buf
    for cfg in wl.CONFIGS:
        if cfg.layers > 1 or (names is not None and cfg.name not in names):
            continue
        t = wl.config_tensors(cfg)
        W0 = t["W"].to(dev)
        x = t["x"].to(dev)
        copies = timing.rotation_copies(W0)
        plan = tp.Plan(cfg.N, cfg.K, cfg.batches)
        for B in cfg.batches:
            y = torch.empty((B, cfg.N), dtype=torch.bfloat16, device=dev)
            xb = x[:B]
            calls = [(lambda W=W: plan.run(xb, W, y)) for W in copies]
            cold = timing.time_calls(calls, warmup=3, reps=60)
            hot = timing.time_calls([lambda: plan.run(xb, W0, y)], warmup=3, reps=30)
            nbytes = wl.algorithmic_bytes(B, cfg.N, cfg.K)
            tac, _ = plan.tactic(B)
            p = {"config": cfg.name, "N": cfg.N, "K": cfg.K, "B": B,
                 "us_median": round(cold["us_median"], 2), "us_p10": round(cold["us_p10"], 2),
                 "us_p90": round(cold["us_p90"], 2), "us_b2b": round(cold["us_mean_b2b"], 2),
                 "GBps": round(timing.gbs(nbytes, cold["us_median"]), 1),
                 "pct_peak": round(100 * timing.gbs(nbytes, cold["us_median"]) / timing.HBM_PEAK_GBS, 1),
                 "hot_us": round(hot["us_median"], 2),
                 "TFLOPs": round(2.0 * B * cfg.N * cfg.K / (cold["us_median"] * 1e-6) / 1e12, 1),
                 "kernel": plan.kernel_name(B), "tactic": tac.as_dict()}
            out["points"].append(p)
            _say(f"{cfg.name:12s} B={B:3d} {p['us_median']:8.2f} us {p['GBps']:8.1f} GB/s "
                 f"{p['pct_peak']:5.1f}% hot {p['hot_us']:7.2f} us  {p['kernel']}")
        del copies, W0, x, t
        torch.cuda.empty_cache()
    if names is not None and "multilayer" not in names:
        with open(args.report, "w") as f:
            json.dump(out, f, indent=1)
        return
    # multi-layer stream: 8 x (in-proj 14560x7168 -> o_proj 7168x12288), B = 64
    cfg = wl.BY_NAME["multilayer"]
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    w_in = [(torch.randn((wl.DSA_N, wl.DSA_K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            for _ in range(cfg.layers)]
    w_o = [(torch.randn((wl.OPROJ_N, wl.OPROJ_K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
           for _ in range(cfg.layers)]
    x0 = torch.randn((cfg.bmax, wl.DSA_K), generator=g, device=dev).to(torch.bfloat16)
    pin = tp.Plan(wl.DSA_N, wl.DSA_K, [cfg.bmax])
    po = tp.Plan(wl.OPROJ_N, wl.OPROJ_K, [cfg.bmax])
    stack = tp.LayerStack(pin, po, w_in, w_o)
    y_in, y_o = stack.buffers(cfg.bmax)
    r = timing.time_calls([lambda: stack.run(x0, y_in, y_o)], warmup=3, reps=20)
    nbytes = cfg.layers * (wl.algorithmic_bytes(cfg.bmax, wl.DSA_N, wl.DSA_K)
                           + wl.algorithmic_bytes(cfg.bmax, wl.OPROJ_N, wl.OPROJ_K))
    out["multilayer"] = {"layers": cfg.layers, "B": cfg.bmax, "us_median": round(r["us_median"], 1),
                         "GBps": round(timing.gbs(nbytes, r["us_median"]), 1),
                         "bytes": nbytes, "in_kernel": pin.kernel_name(cfg.bmax),
                         "o_kernel": po.kernel_name(cfg.bmax)}
    # the same chain captured once as a graph and replayed (the launches of
    # all 2 x 8 projections, split-K passes included, submitted as one)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stack.run(x0, y_in, y_o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack.run(x0, y_in, y_o)
    torch.cuda.synchronize()
    rg = timing.time_calls([graph.replay], warmup=3, reps=20)
    out["multilayer"].update({"graph_us_median": round(rg["us_median"], 1),
                              "graph_GBps": round(timing.gbs(nbytes, rg["us_median"]), 1)})
    del graph
    _say(f"multilayer 8x(in+o) B=64: {out['multilayer']}")
    with open(args.report, "w") as f:
        json.dump(out, f, indent=1)
    return out


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
    if args.report and args.configs:
        # a report of selected configurations only (e.g. under a counter run):
        # no headline steps, so every dispatch belongs to the named points
        report(args, torch, tp, wl, timing)
        return
    h = headline(args, torch, tp, wl, timing)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, h["cfg"], h["t"], wl)
    if args.report:
        report(args, torch, tp, wl, timing)
    if args.copy_calibration:
        copy_calibration(torch)
    cfg = h["cfg"]
    line = {
        "metric": "achieved HBM GB/s (algorithmic W+x+y bytes / time), TP1 BF16 decode "
                  "projection, o_proj sweep",
        "value": round(h["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_seconds": args.warm_seconds,
        "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "o_proj sweep: W 7168x12288 BF16 ~N(0,0.02), x[B,12288] ~N(0,1), "
                               "B in {1,2,4,8,16}, seed 1; one call per B per step",
                   "N": cfg.N, "K": cfg.K, "batches": list(cfg.batches),
                   "weight_copies": h["copies"], "step_bytes": h["step_bytes"]},
        "per_batch_us": {str(B): r["us_per_call"] for B, r in h["per_b"].items()},
        "per_batch_GBps": {str(B): r["GBps"] for B, r in h["per_b"].items()},
        "kernels": {str(B): r["kernel"] for B, r in h["per_b"].items()},
        "roofline": h["roofline"],
        "read_ceiling": h["read_ceiling"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
