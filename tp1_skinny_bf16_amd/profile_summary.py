"""Summarise rocprofv3 CSV output of a bench run into profiles/.

Reads the directories written by
  rocprofv3 --kernel-trace --stats -f csv -d <kt>    -o kt -- python bench.py ... --copy-calibration
  rocprofv3 --pmc FETCH_SIZE       -f csv -d <fetch> -o f  -- python bench.py ... --copy-calibration
  rocprofv3 --pmc WRITE_SIZE       -f csv -d <write> -o w  -- python bench.py ... --copy-calibration
and writes
  <out>/<name>_kernel_trace.md  average kernel durations (the projection kernels
                                and the 256 MiB reference copy)
  <out>/<name>_traffic.md       FETCH_SIZE / WRITE_SIZE per dispatch, scaled by
                                what the same counter reads for the reference
                                copy of known size, against algorithmic bytes
  <out>/traffic.json            per-kernel scaled bytes (by name, and by
                                name@grid work-items), tagged with the hash of
                                the kernel source they were taken from
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(PKG, "csrc", "kernels.hip")
COPY_BYTES = 268435456  # the reference copy reads and writes this many bytes
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def short(name: str) -> str:
    """'void tp1::stream_kernel<1, 4, 4, true>(tp1::StreamArgs)' -> 'stream_kernel<1, 4, 4, true>'"""
    n = name.replace("void ", "").split("(")[0]
    return n.replace("tp1::", "")


def counters(d):
    """Mean and largest counter value per dispatch, by kernel name and by
    (name, grid size in work-items): one kernel (the split-K pass) serves
    several shapes, which only its grid tells apart."""
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    per = collections.defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        per[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return ({k: sum(v) / len(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()},
            {k: max(v) for k, v in per.items()})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--kt", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--bench-json", required=True, help="the bench.py JSON line of the run")
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True, help="the command lines that made the data")
    ap.add_argument("--out", default="profiles")
    a = ap.parse_args()

    line = json.loads(open(a.bench_json).read().strip().splitlines()[-1])
    algo = {}  # kernel short name -> algorithmic bytes per launch (mean over its uses)
    from workloads import algorithmic_bytes  # noqa: E402  (repo root on sys.path)
    per_kernel = collections.defaultdict(list)
    # the multi-layer stream's two projections (bench.py default / --headline-only)
    for fam in (line.get("kernels") or {}).values():
        per_kernel[fam["kernel"].split("+")[0]].append(fam["bytes_per_launch"])
    # the single-projection workloads (bench.py per_config / --sweeps-only)
    for cfg in (line.get("per_config") or {}).values():
        for B, pt in cfg["points"].items():
            per_kernel[pt["kernel"].split("+")[0]].append(
                algorithmic_bytes(int(B), cfg["N"], cfg["K"]))
    # the MoE front's one-launch calls (bench.py moe_front / --front-only)
    for pt in ((line.get("moe_front") or {}).get("points") or []):
        per_kernel[pt["kernel"].split("+")[0]].append(algorithmic_bytes(pt["B"], pt["N"], pt["K"]))
    for k, v in per_kernel.items():
        algo[k] = sum(v) / len(v)

    stats = list(csv.DictReader(open(_one(os.path.join(a.kt, "**", "*kernel_stats.csv")))))
    fetch, nf, fmax = counters(a.fetch)
    write, nw, wmax = counters(a.write)
    # The reference copy: the copy kernel's dispatches that fetch the most.
    # Any other device copy of the run (a smaller one, possibly with the same
    # grid, such as the packing of a weight) fetches less, so the largest
    # value per dispatch is the reference's.
    copy_key = max((k for k in fetch if not isinstance(k, str) and COPY_KERNEL in k[0]),
                   key=lambda k: fmax[k])
    copy_fetch, copy_write = fmax[copy_key], wmax[copy_key]
    f_scale = copy_fetch * 1024 / COPY_BYTES
    w_scale = copy_write * 1024 / COPY_BYTES

    os.makedirs(a.out, exist_ok=True)
    kt = [f"# Kernel trace: {a.name}", "", "Command:", "", "```", a.command, "```", "",
          "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        nm = r["Name"]
        if "tp1::" in nm or COPY_KERNEL in nm:
            kt.append(f"| `{short(nm)}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                      f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    kt += ["", f"Reference copy: {COPY_BYTES} bytes read and written per call."]
    with open(os.path.join(a.out, f"{a.name}_kernel_trace.md"), "w") as f:
        f.write("\n".join(kt) + "\n")

    tr = [f"# HBM traffic: {a.name}", "", "Command:", "", "```", a.command, "```", "",
          f"Scale: the reference copy reads and writes {COPY_BYTES} bytes; per dispatch "
          f"(grid {copy_key[1]}, the largest of its {nf[copy_key]} copy dispatches) FETCH_SIZE "
          f"reads {copy_fetch:.1f} KiB and WRITE_SIZE {copy_write:.1f} KiB, "
          f"so bytes = FETCH_SIZE KiB * 1024 / {f_scale:.5f} and "
          f"WRITE_SIZE KiB * 1024 / {w_scale:.5f}.", "",
          "| kernel | grid (work-items) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB "
          "| scaled read MB | scaled write MB | algorithmic MB | traffic / algorithmic |",
          "|---|---|---|---|---|---|---|---|---|"]
    out = {"source_hash": source_hash(), "kernels": {}}
    grids = collections.Counter(k[0] for k in fetch if not isinstance(k, str))
    for k in fetch:
        name = k if isinstance(k, str) else k[0]
        if "tp1::" not in name:
            continue
        s = short(name) if isinstance(k, str) else f"{short(name)}@{k[1]}"
        rd = fetch[k] * 1024 / f_scale
        wr = write.get(k, 0.0) * 1024 / w_scale
        out["kernels"][s] = {"read_bytes": rd, "write_bytes": wr, "traffic": rd + wr}
        if isinstance(k, str):
            continue                      # the table lists one row per (kernel, grid)
        al = algo.get(short(name)) if grids[name] == 1 else None
        ratio = f"{(rd + wr) / al:.3f}" if al else "-"
        tr.append(f"| `{short(name)}` | {k[1]} | {nf[k]} | {fetch[k]:.1f} | "
                  f"{write.get(k, 0.0):.1f} | {rd / 1e6:.2f} | {wr / 1e6:.3f} | "
                  f"{al / 1e6 if al else 0:.2f} | {ratio} |")
    with open(os.path.join(a.out, f"{a.name}_traffic.md"), "w") as f:
        f.write("\n".join(tr) + "\n")
    path = os.path.join(a.out, "traffic.json")
    prev = json.load(open(path)) if os.path.exists(path) else {}
    if prev.get("source_hash") == out["source_hash"]:
        prev["kernels"].update(out["kernels"])
        out = prev
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(kt + [""] + tr))


if __name__ == "__main__":
    main()
