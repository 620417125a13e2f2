"""Summarise a rocprofv3 --pmc run of the projection kernels into a table.

    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE ... \\
        -f csv -d <dir> -o p -- python bench.py --report <json> --configs dsa_sweep --no-cpu
    python -m tp1_skinny_bf16_amd.counter_summary --dir <dir> [<dir> ...] --name <name> \\
        --command "<the commands>" [--cus 256]

Per kernel instance (name and grid size) it lists the mean of every counter
over its dispatches, and, when SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
were collected, the MFMA busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / ((GRBM_GUI_ACTIVE / XCDs) * compute units * 4 SIMDs).
GRBM_GUI_ACTIVE comes summed over the XCDs (divided by 8 it matches the
dispatch's duration at the shader clock), SQ_VALU_MFMA_BUSY_CYCLES over
the compute units.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import os


def short(name: str) -> str:
    return name.replace("void ", "").split("(")[0].replace("tp1::", "")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--dir", required=True, nargs="+",
                    help="one directory per --pmc pass (their counters are merged)")
    ap.add_argument("--name", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--out", default="profiles")
    a = ap.parse_args()
    files = sorted(f for d in a.dir
                   for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                      recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {a.dir}")
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in files:
        for r in csv.DictReader(open(path)):
            if "tp1::" not in r["Kernel_Name"]:
                continue
            key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    counters = sorted({c for v in vals.values() for c in v})
    mfma = "SQ_VALU_MFMA_BUSY_CYCLES" in counters and "GRBM_GUI_ACTIVE" in counters
    l2 = "TCC_HIT_sum" in counters and "TCC_MISS_sum" in counters
    head = ["kernel", "grid", "dispatches"] + counters + (["MFMA busy"] if mfma else []) + \
        (["L2 hit"] if l2 else [])
    lines = [f"# Counters: {a.name}", "", "Command:", "", "```", a.command, "```", "",
             "| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for (k, grid), v in sorted(vals.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        n = max(len(x) for x in v.values())
        row = [f"`{k}`", str(grid), str(n)]
        means = {c: sum(v[c]) / len(v[c]) for c in v}
        row += [f"{means[c]:.4g}" if c in means else "-" for c in counters]
        if mfma:
            active = means["GRBM_GUI_ACTIVE"] / a.xcds
            busy = means["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * a.cus * 4)
            row.append(f"{100 * busy:.1f}%")
        if l2:
            req = means["TCC_HIT_sum"] + means["TCC_MISS_sum"]
            row.append(f"{100 * means['TCC_HIT_sum'] / req:.1f}%" if req else "-")
        lines.append("| " + " | ".join(row) + " |")
    if mfma:
        lines += ["", f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ((GRBM_GUI_ACTIVE / {a.xcds} XCDs) "
                      f"x {a.cus} compute units x 4 SIMDs), per dispatch.  GRBM_GUI_ACTIVE is "
                      f"summed over the XCDs: divided by {a.xcds} it is the dispatch's duration "
                      "in shader clocks."]
    if l2:
        lines += ["", "L2 hit = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum), per dispatch: the "
                      "share of the kernel's L2 requests served by L2 (x, re-read by every "
                      "workgroup, hits; the weight, streamed once, misses)."]
    os.makedirs(a.out, exist_ok=True)
    with open(os.path.join(a.out, f"{a.name}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
