"""Render rocprofv3 --kernel-trace --stats output as a short Markdown table
(the summaries kept under profiles/)."""
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
        name = r["Name"].split("(")[0].replace("void ", "")
        out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    stats_dir, title, command, out = sys.argv[1:5]
    note = sys.argv[5] if len(sys.argv) > 5 else ""
    open(out, "w").write(kernel_table(stats_dir, title, command, note))
    print(open(out).read())
