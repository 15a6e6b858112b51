"""Format a rocprofv3 ``--stats`` kernel summary (``*_kernel_stats.csv``) as a short text table.

    python -m sequence_mixing_amd.profsum <kernel_stats.csv> "<command that produced it>" [title]
"""
from __future__ import annotations

import csv
import sys


def summarize(path: str, command: str, title: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    lines = [f"# {title}" if title else "# rocprofv3 kernel summary", "", f"command: {command}", "",
             f"{'kernel':<72} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total%':>7}"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        name = name.split("(")[0] if not name.startswith("void at::") else name[:60]
        lines.append(f"{name[:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>9.2f} "
                     f"{float(r['MinNs'])/1e3:>9.2f} {float(r['MaxNs'])/1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    print(summarize(sys.argv[1], sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""), end="")
