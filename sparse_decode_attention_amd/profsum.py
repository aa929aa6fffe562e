"""Render rocprofv3 output as short Markdown tables (the summaries kept under
profiles/): kernel durations from --kernel-trace --stats, and per-dispatch
counter averages from --pmc runs."""
from __future__ import annotations

import csv
import glob
import os
import sys


def kernel_table(stats_dir: str, title: str, command: str, note: str = "", match: str = "spark::") -> str:
    rows = []
    for f in glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    keep = [r for r in rows if match in r["Name"] or "copyBuffer" in r["Name"]]
    keep.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {title}", "", "Command:", "", f"    {command}", ""]
    if note:
        out += [note, ""]
    out += ["| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in keep:
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def counter_means(pmc_dir: str, match: str) -> dict:
    """Per kernel whose name contains `match`: each counter summed over its
    dimension entries within a dispatch, then averaged over dispatches."""
    per = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if match not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per.setdefault(name, {}).setdefault(key, 0.0)
            per[name][key] += float(r["Counter_Value"])
    out = {}
    for name, d in per.items():
        acc = {}
        for (_, c), v in d.items():
            acc.setdefault(c, []).append(v)
        out[name] = {c: sum(v) / len(v) for c, v in acc.items()}
    return out


def counter_table(runs: list, counters: list, title: str, note: str = "") -> str:
    """runs: (label, pmc_dir, kernel-name match, command) per column."""
    cols = []
    for label, d, match, _ in runs:
        means = counter_means(d, match)
        if len(means) != 1:
            raise ValueError(f"{d}: {len(means)} kernels match {match!r}")
        cols.append((label, *next(iter(means.items()))))
    out = [f"# {title}", ""]
    for label, _, _, cmd in runs:
        out += [f"Command ({label}):", "", f"    {cmd}", ""]
    if note:
        out += [note, ""]
    out += ["| counter (per dispatch) | " + " | ".join(f"{lab}: {k}" for lab, k, _ in cols) + " |",
            "|---|" + "---|" * len(cols)]
    for c in counters:
        out.append(f"| {c} | " + " | ".join(f"{v.get(c, float('nan')):.0f}" for _, _, v in cols) + " |")
    waves = [v.get("SQ_WAVES") for _, _, v in cols]
    if all(waves):
        for c in counters:
            if c.startswith("SQ_INSTS_"):
                out.append(f"| {c} per wave | " + " | ".join(f"{v.get(c, 0) / v['SQ_WAVES']:.1f}" for _, _, v in cols)
                           + " |")
    return "\n".join(out) + "\n"


def kernel_counter_table(pmc_dir: str, counters: list, title: str, command: str, note: str = "",
                         match: str = "spark::") -> str:
    """One row per kernel of a --pmc run: each counter per dispatch (summed
    over its dimension entries, averaged over dispatches), then the
    instruction counts per wave."""
    means = counter_means(pmc_dir, match)
    out = [f"# {title}", "", "Command:", "", f"    {command}", ""]
    if note:
        out += [note, ""]
    inst = [c for c in counters if c.startswith("SQ_INSTS_")]
    head = ["kernel"] + counters + [f"{c[9:]} / wave" for c in inst]
    out += ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for name in sorted(means, key=lambda n: -means[n].get("SQ_WAVES", 0)):
        m = means[name]
        waves = m.get("SQ_WAVES", 0)
        row = [name.replace("spark::", "")] + [f"{m.get(c, float('nan')):.0f}" for c in counters]
        row += [f"{m.get(c, 0) / waves:.0f}" if waves else "" for c in inst]
        out.append("| " + " | ".join(row) + " |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    stats_dir, title, command, out = sys.argv[1:5]
    note = sys.argv[5] if len(sys.argv) > 5 else ""
    open(out, "w").write(kernel_table(stats_dir, title, command, note))
    print(open(out).read())
