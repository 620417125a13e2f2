"""Tactic measurement: time candidate tactics per (N, K, batch bin) on the GPU
and pick the table the library ships (tactics_table.cpp).

The vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep"
keeps per-batch tactic tables for its projections (its opening text names
DEP_PROJECTION and DEP_OPROJ; section "_bins" gives the lookup rule); this
tool builds the MI355X one by measurement.  Each candidate
is timed over rotated weight copies (>= 1 GB, so every call streams its
weight from HBM).  The time ranked is the mean per call of `reps` calls
enqueued back to back (how a decode step issues its projections, and where a
split-K call pays its second launch in full); the median of per-call event
timings is kept beside it.  With --graph the same `reps` calls are captured
in one graph and replayed, so that the host's launch submission (~6 us per
call through the binding) does not bound kernels that short; the small
tensor-parallel shards are tuned that way.  Ties within 1% go to fewer
launches (no split-K pass), then the smaller split, then fewer rows per wave.
The crossover is the smallest batch whose best tactic is an MFMA one.

    python -m tp1_skinny_bf16_amd.tune --shape 14560x7168 --bins 1,2,4 --out t.json

A run made on another box than the table's may differ from it by a few
percent everywhere, so a table change is decided on one box:

    python -m tp1_skinny_bf16_amd.tune --recheck t.json --out r.json

times every bin whose run choice beat the table's tactic (in that run) by more
than --margin against it again, in --pairs alternating pairs.
"""
from __future__ import annotations

import argparse
import itertools
import json
import sys
import time

import torch

from . import (KERNEL_IDS, KERNEL_MFMA_PIPE, KERNEL_MFMA_XS, KERNEL_STREAM,
               KERNEL_STREAM_DOT2, Plan, ProjError, Tactic)
from .timing import gbs, rotation_copies, time_calls, time_graph

SHAPES = {"dsa": (14560, 7168), "oproj": (7168, 12288), "kda": (49376, 7168)}


def next_pow2(v: int) -> int:
    p = 1
    while p < v:
        p <<= 1
    return p


def candidates(bin_: int, full: bool = False):
    out = []
    if bin_ <= 8:
        bc = next_pow2(bin_)
        for kern, rows, split, waves, wpc in itertools.product(
                (KERNEL_STREAM, KERNEL_STREAM_DOT2), (1, 2, 4), (1, 2, 3, 4),
                (1, 2, 4, 8), (2, 4, 6, 8, 12, 16)):
            if not full and (waves == 8 and wpc < 8 or split > 2):
                continue
            out.append(Tactic(kern, bc, split, rows, waves, wpc))
    bc = max(16, next_pow2(bin_))
    xs = {16: ((4, 1, 128, 1), (4, 1, 128, 2), (4, 1, 256, 2), (4, 1, 512, 1), (8, 1, 128, 1),
               (8, 1, 128, 2), (8, 1, 256, 1), (16, 1, 128, 1)),
          32: ((4, 1, 128, 1), (4, 1, 128, 2), (4, 2, 128, 1), (8, 2, 128, 1), (8, 2, 256, 1)),
          64: ((4, 1, 128, 1), (4, 2, 128, 1), (4, 2, 128, 2), (4, 4, 128, 1), (8, 2, 128, 1),
               (8, 2, 256, 1)),
          128: ((4, 2, 128, 1), (4, 4, 128, 1)), 256: ((4, 4, 128, 1), (2, 4, 128, 1))}[bc]
    for (rows, waves, kc, depth), split, wpc in itertools.product(xs, (1, 2, 3, 4), (1, 2)):
        out.append(Tactic(KERNEL_MFMA_XS, bc, split, rows, waves, wpc, kc, depth))
        if split <= 2:
            out.append(Tactic(KERNEL_MFMA_XS, bc, split, rows, waves, wpc, kc, depth,
                              stagger=1))
    pipe = {16: ((4, 1, 1, 128, 3, 4), (4, 1, 1, 128, 4, 4), (4, 1, 1, 128, 6, 4),
                 (4, 1, 1, 256, 3, 4), (8, 1, 1, 128, 3, 4), (8, 1, 1, 128, 4, 4),
                 (2, 1, 2, 256, 6, 4), (2, 1, 2, 256, 4, 4), (2, 1, 2, 128, 8, 4),
                 (1, 1, 4, 256, 4, 4), (1, 1, 4, 256, 6, 4), (8, 1, 1, 256, 2, 8),
                 (4, 1, 2, 256, 3, 8), (2, 1, 4, 256, 6, 8),
                 (2, 1, 4, 256, 4, 8), (1, 1, 8, 256, 4, 8), (2, 1, 4, 512, 3, 8),
                 (2, 1, 4, 512, 2, 8), (1, 1, 8, 512, 4, 8), (2, 1, 4, 512, 3, 4),
                 (1, 1, 8, 512, 3, 8)),
            32: ((4, 1, 1, 128, 4, 4), (4, 1, 1, 128, 6, 4), (4, 2, 1, 64, 8, 4),
                 (8, 2, 1, 128, 3, 4), (2, 1, 2, 256, 4, 4), (2, 2, 1, 256, 4, 4),
                 (8, 2, 1, 128, 3, 8), (2, 1, 4, 256, 4, 8), (4, 2, 1, 128, 4, 8),
                 (4, 1, 2, 128, 4, 8), (4, 1, 2, 256, 3, 8), (2, 2, 2, 256, 4, 8)),
            64: ((4, 2, 1, 64, 8, 4), (4, 2, 1, 128, 4, 4), (4, 4, 1, 64, 8, 4),
                 (8, 2, 1, 64, 4, 4), (8, 2, 1, 64, 6, 4), (16, 2, 1, 64, 3, 8),
                 (8, 2, 1, 128, 3, 8), (16, 1, 1, 64, 3, 8), (8, 4, 1, 128, 3, 8),
                 (8, 2, 1, 64, 6, 8), (4, 2, 1, 128, 4, 8), (4, 2, 2, 128, 4, 8),
                 (4, 4, 1, 128, 4, 8), (4, 2, 1, 256, 2, 8), (2, 4, 1, 128, 4, 8),
                 (2, 2, 2, 128, 4, 8)),
            128: ((4, 4, 1, 64, 6, 4), (4, 4, 1, 32, 12, 4), (8, 4, 1, 64, 4, 4),
                  (8, 4, 1, 32, 8, 4), (16, 2, 1, 64, 3, 8), (8, 2, 1, 64, 4, 8),
                  (16, 4, 1, 32, 4, 8), (8, 2, 1, 32, 8, 8), (16, 2, 1, 32, 6, 8),
                  (4, 2, 1, 64, 4, 8), (4, 4, 1, 64, 4, 8)),
            256: ((4, 4, 1, 32, 7, 4), (4, 4, 1, 64, 3, 4), (8, 4, 1, 32, 6, 4),
                  (8, 4, 1, 64, 3, 4), (16, 4, 1, 32, 4, 8),
                  (8, 4, 1, 64, 3, 8), (8, 8, 1, 64, 3, 8), (8, 4, 1, 32, 6, 8))}[bc]
    for (rows, waves, kw, kc, depth, nw), split, wpc in itertools.product(
            pipe, (1, 2, 3, 4, 6, 8), (1, 2)):
        if (split > 4 and bc < 64) or (nw == 8 and wpc > 1):
            continue
        out.append(Tactic(KERNEL_MFMA_PIPE, bc, split, rows, waves, wpc, kc, depth, kw, nw))
        if split in (1, 2, 4):
            out.append(Tactic(KERNEL_MFMA_PIPE, bc, split, rows, waves, wpc, kc, depth, kw, nw,
                              stagger=1))
    return out


def _key(res):
    t = res["tactic"]
    return (res["us"], t["split"] > 1, t["split"], t["rows"])


def measure(N: int, K: int, bins, reps: int = 40, log=None, full: bool = False,
            fused_split: bool = False, graph: bool = False, only=None):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    W0 = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    copies = rotation_copies(W0)
    bmax = max(bins)
    x = torch.randn((bmax, K), generator=g, device=dev).to(torch.bfloat16)
    plan = Plan(N, K, bins, fused_split=fused_split)
    result = {"N": N, "K": K, "copies": len(copies), "bins": {}, "fused_split": fused_split,
              "graph": graph}
    # half a second of the default tactic first: the first timings of a cold
    # process otherwise run at ramping clocks
    y0 = torch.empty((bins[0], N), dtype=torch.bfloat16, device=dev)
    st0 = torch.cuda.current_stream().cuda_stream
    t_end = time.time() + 0.5
    while time.time() < t_end:
        for W in copies:
            plan.run_ptr(bins[0], x.data_ptr(), K, W.data_ptr(), y0.data_ptr(), st0)
        torch.cuda.synchronize()
    for b in bins:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=dev)
        xb = x[:b]
        st = torch.cuda.current_stream().cuda_stream
        rows = []
        cands = candidates(b, full)
        if only:
            # a subset of the kernel families, measured beside the tactic the
            # library's table gives this bin
            table_t, _ = Plan(N, K, bins, host_only=True).tactic(b)
            cands = [table_t] + [t for t in cands if t.kernel_name in only and t != table_t]
        for t in cands:
            try:
                plan.set_tactic(b, t)
            except ProjError:
                continue
            if graph:
                # `reps` calls round-robin over the copies, captured in one
                # graph; each call launches on the current (capture) stream
                gcalls = [(lambda W=copies[i % len(copies)]: plan.run_ptr(
                    b, xb.data_ptr(), K, W.data_ptr(), y.data_ptr(),
                    torch.cuda.current_stream().cuda_stream)) for i in range(reps)]
                us = time_graph(gcalls)
                rows.append({"tactic": t.as_dict(), "us": round(us, 2), "us_call": None,
                             "kernel": plan.kernel_name(b)})
                continue
            calls = [(lambda W=W: plan.run_ptr(b, xb.data_ptr(), K, W.data_ptr(),
                                               y.data_ptr(), st)) for W in copies]
            r = time_calls(calls, warmup=2, reps=reps, warm_seconds=0.0)
            # ranked by the back-to-back mean: projections run queued one after
            # another on a stream, where a split-K call pays its second launch
            # in full; the per-call median (own event pair) is kept beside it
            rows.append({"tactic": t.as_dict(), "us": round(r["us_mean_b2b"], 2),
                         "us_call": round(r["us_median"], 2), "kernel": plan.kernel_name(b)})
        rows.sort(key=_key)
        best = rows[0]
        # ties within 1%: prefer no split pass, then smaller split, fewer rows
        near = [r for r in rows if r["us"] <= best["us"] * 1.01]
        near.sort(key=lambda r: (r["tactic"]["split"] > 1, r["tactic"]["split"],
                                 r["tactic"]["rows"], r["us"]))
        chosen = near[0]
        nbytes = 2 * N * K + 2 * b * K + 2 * b * N
        result["bins"][b] = {"chosen": chosen, "GBps": round(gbs(nbytes, chosen["us"]), 1),
                             "top": rows[:8], "all": rows, "n_candidates": len(rows)}
        best_stream = min((r for r in rows if r["tactic"]["kernel"].startswith("stream")),
                          key=lambda r: r["us"], default=None)
        best_mfma = min((r for r in rows if r["tactic"]["kernel"].startswith("mfma")),
                        key=lambda r: r["us"], default=None)
        result["bins"][b]["best_stream_us"] = best_stream["us"] if best_stream else None
        result["bins"][b]["best_mfma_us"] = best_mfma["us"] if best_mfma else None
        if log:
            log(f"{N}x{K} B={b}: {chosen['us']:.2f} us {result['bins'][b]['GBps']} GB/s "
                f"{chosen['kernel']} {chosen['tactic']} (stream {result['bins'][b]['best_stream_us']}"
                f" / mfma {result['bins'][b]['best_mfma_us']}, {len(rows)} candidates)")
        plan.set_tactic(b, Tactic(**{**chosen["tactic"],
                                     "kernel": KERNEL_IDS[chosen["tactic"]["kernel"]]}))
    mfma_bins = [b for b in bins
                 if result["bins"][b]["chosen"]["tactic"]["kernel"].startswith("mfma")]
    result["crossover"] = min(mfma_bins) if mfma_bins else None
    return result


def table_rows(result) -> str:
    lines = []
    for b, r in result["bins"].items():
        t = dict(r["chosen"]["tactic"])
        if t["kernel"] == "mfma_pipe" and not t.get("kw"):
            t["kw"] = 1  # measured before the field existed: one wave along K
        if t["kernel"] == "mfma_pipe" and not t.get("nw"):
            t["nw"] = 4  # measured before the field existed: four waves
        k = {"stream": "PROJ_KERNEL_STREAM", "stream_dot2": "PROJ_KERNEL_STREAM_DOT2",
             "mfma_xs": "PROJ_KERNEL_MFMA_XS", "mfma_pipe": "PROJ_KERNEL_MFMA_PIPE"}[t["kernel"]]
        lines.append(f"    {{{result['N']}, {result['K']}, {b}, {{{k}, {t['bcap']}, {t['split']}, "
                     f"{t['rows']}, {t['waves']}, {t['wpc']}, {t.get('kc', 0)}, "
                     f"{t.get('depth', 0)}, {t.get('kw', 0)}, {t.get('nw', 0)}, "
                     f"{t.get('stagger', 0)}}}}},  // "
                     f"{r['chosen']['us']} us, {r['GBps']} GB/s")
    return "\n".join(lines)


def emit_table(paths) -> str:
    """C++ rows of tactics_table.cpp from tuner JSON files: per (N, K, bin)
    the fastest chosen tactic over the runs given (runs on different boxes
    differ by a few percent, so no single run is the reference)."""
    chosen = {}
    for path in paths:
        with open(path) as f:
            for res in json.load(f):
                for b, r in res["bins"].items():
                    key = (res["N"], res["K"], int(b))
                    if key not in chosen or r["chosen"]["us"] < chosen[key]["chosen"]["us"]:
                        chosen[key] = r
    merged = {}
    for (N, K, b), r in chosen.items():
        merged.setdefault((N, K), {"N": N, "K": K, "bins": {}})["bins"][b] = r
    out = []
    for key in sorted(merged):
        res = merged[key]
        res["bins"] = dict(sorted(res["bins"].items()))
        out.append(table_rows(res))
    return "\n".join(out)


def summarize(paths) -> str:
    """Markdown of the measured tables: chosen tactic per bin, the best stream
    and best MFMA candidate, and the crossover (per bin the fastest run, as
    emit_table picks it)."""
    chosen = {}
    for path in paths:
        with open(path) as f:
            for res in json.load(f):
                for b, r in res["bins"].items():
                    key = (res["N"], res["K"], int(b))
                    if key not in chosen or r["chosen"]["us"] < chosen[key]["chosen"]["us"]:
                        chosen[key] = r
    lines = []
    for (N, K) in sorted({(n, k) for n, k, _ in chosen}):
        bins = sorted(b for n, k, b in chosen if (n, k) == (N, K))
        lines += [f"## {N} x {K}", "",
                  "| bin | chosen kernel | tactic (bcap, split, rows, waves, wpc, kc, depth, kw, nw, "
                  "stagger) "
                  "| us "
                  "| GB/s "
                  "| best stream us | best MFMA us | candidates |",
                  "|---|---|---|---|---|---|---|---|"]
        cross = None
        for b in bins:
            r = chosen[(N, K, b)]
            t = r["chosen"]["tactic"]
            if cross is None and t["kernel"].startswith("mfma"):
                cross = b
            lines.append(f"| {b} | `{r['chosen']['kernel']}` | {t['bcap']}, {t['split']}, {t['rows']}, "
                         f"{t['waves']}, {t['wpc']}, {t.get('kc', 0)}, {t.get('depth', 0)}, "
                         f"{t.get('kw', 0)}, {t.get('nw', 0)}, {t.get('stagger', 0)} | "
                         f"{r['chosen']['us']} | {r['GBps']} | "
                         f"{r.get('best_stream_us')} | {r.get('best_mfma_us')} | {r['n_candidates']} |")
        lines += ["", f"Crossover (first bin whose best tactic is an MFMA kernel): {cross}", ""]
    return "\n".join(lines)


def _tactic_from(d: dict) -> Tactic:
    return Tactic(**{**d, "kernel": KERNEL_IDS[d["kernel"]]})


def recheck_candidates(run, table_tactic, margin: float):
    """(N, K, bin, table tactic, run's choice) for every bin of a tuning run
    whose choice beat the table's tactic, timed in the same run, by more than
    `margin` (a fraction).  table_tactic(N, K, bin) -> Tactic."""
    out = []
    for res in run:
        for b, r in res["bins"].items():
            t = table_tactic(res["N"], res["K"], int(b))
            td = t.as_dict()
            same = next((row["us"] for row in r["all"]
                         if {k: row["tactic"].get(k, 0) for k in td} == td), None)
            best = r["chosen"]
            if same is not None and best["us"] < same * (1.0 - margin):
                out.append((res["N"], res["K"], int(b), t, _tactic_from(best["tactic"])))
    return out


def recheck(paths, margin: float = 0.015, pairs: int = 3, reps: int = 60, log=print):
    """Time each bin's table tactic against a tuning run's choice in
    alternating pairs on one box, so that box-to-box differences between
    runs cannot decide the table.  Returns one row per re-checked bin."""
    run = []
    for path in paths:
        with open(path) as f:
            run += json.load(f)

    def table_tactic(N, K, b):
        return Plan(N, K, [b], host_only=True).tactic(b)[0]

    cands = recheck_candidates(run, table_tactic, margin)
    dev = torch.device("cuda:0")
    rows, shape, copies, x = [], None, None, None
    for (N, K, b, t_tab, t_new) in cands:
        if shape != (N, K):
            copies = None
            torch.cuda.empty_cache()
            g = torch.Generator(device=dev)
            g.manual_seed(7)
            W0 = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            copies = rotation_copies(W0)
            x = torch.randn((256, K), generator=g, device=dev).to(torch.bfloat16)
            shape = (N, K)
        y = torch.empty((b, N), dtype=torch.bfloat16, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        plans = {}
        for name, t in (("table", t_tab), ("run", t_new)):
            plans[name] = Plan(N, K, [b])
            plans[name].set_tactic(b, t)
        us = {"table": [], "run": []}
        for _ in range(pairs):
            for name in ("table", "run"):
                pl = plans[name]
                calls = [(lambda W=W, pl=pl: pl.run_ptr(b, x.data_ptr(), K, W.data_ptr(),
                                                      y.data_ptr(), st)) for W in copies]
                us[name].append(round(time_calls(calls, warmup=2, reps=reps,
                                                  warm_seconds=0.1)["us_mean_b2b"], 2))
        med = {k: sorted(v)[len(v) // 2] for k, v in us.items()}
        row = {"N": N, "K": K, "bin": b, "table": t_tab.as_dict(), "run": t_new.as_dict(),
               "table_us": us["table"], "run_us": us["run"],
               "gain_pct": round(100.0 * (med["table"] - med["run"]) / med["table"], 2)}
        rows.append(row)
        if log:
            log(f"{N}x{K} B={b}: table {us['table']} run {us['run']} -> {row['gain_pct']}%")
    return rows


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--recheck":
        ap = argparse.ArgumentParser(prog="tune --recheck")
        ap.add_argument("--recheck", nargs="+", required=True, help="tuning run JSON files")
        ap.add_argument("--margin", type=float, default=0.015)
        ap.add_argument("--pairs", type=int, default=3)
        ap.add_argument("--out", required=True)
        a = ap.parse_args()
        rows = recheck(a.recheck, a.margin, a.pairs, log=lambda m: print(m, flush=True))
        with open(a.out, "w") as f:
            json.dump(rows, f, indent=1)
        return 0
    if len(sys.argv) > 1 and sys.argv[1] == "--emit-table":
        print(emit_table(sys.argv[2:]))
        return 0
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        print(summarize(sys.argv[2:]))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--shape", action="append", required=True,
                    help="NxK or one of " + ",".join(SHAPES))
    ap.add_argument("--bins", default="1,2,4,8,16,32,64,128,256")
    ap.add_argument("--reps", type=int, default=40)
    ap.add_argument("--full", action="store_true")
    ap.add_argument("--fused-split", action="store_true",
                    help="measure with the in-kernel split-K reduction")
    ap.add_argument("--graph", action="store_true",
                    help="time each candidate's calls captured in one graph (for kernels "
                         "as short as the host's launch submission)")
    ap.add_argument("--only", default=None,
                    help="comma-separated kernel families to measure (e.g. mfma_pipe), beside "
                         "the table's tactic for each bin")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    bins = [int(v) for v in a.bins.split(",")]
    allres = []
    t0 = time.time()
    for sh in a.shape:
        N, K = SHAPES[sh] if sh in SHAPES else (int(v) for v in sh.split("x"))
        res = measure(N, K, bins, a.reps, log=lambda m: print(m, flush=True), full=a.full,
                      fused_split=a.fused_split, graph=a.graph,
                      only=set(a.only.split(",")) if a.only else None)
        allres.append(res)
        print(table_rows(res), flush=True)
        print(f"crossover (first MFMA bin) for {N}x{K}: {res['crossover']}  "
              f"[{time.time() - t0:.0f} s]", flush=True)
        with open(a.out, "w") as f:
            json.dump(allres, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
