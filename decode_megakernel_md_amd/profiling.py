"""Profiling helpers: summarise rocprofv3 output.

    python -m decode_megakernel_md_amd.profiling <kernel_stats.csv | results.db>

prints a per-kernel table (calls, total/avg/min/max duration in microseconds)
from either rocprofv3's --stats CSV or its rocpd SQLite database."""
from __future__ import annotations

import csv
import sqlite3
import sys
from typing import Dict, List


def stats_from_db(path: str) -> List[Dict]:
    db = sqlite3.connect(path)
    rows = db.execute("select name, count(*), sum(duration), avg(duration), min(duration), max(duration) "
                      "from kernels group by name order by sum(duration) desc").fetchall()
    return [{"name": r[0], "calls": r[1], "total_us": r[2] / 1e3, "avg_us": r[3] / 1e3, "min_us": r[4] / 1e3,
             "max_us": r[5] / 1e3} for r in rows]


def stats_from_csv(path: str) -> List[Dict]:
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append({"name": r["Name"], "calls": int(r["Calls"]), "total_us": float(r["TotalDurationNs"]) / 1e3,
                        "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                        "max_us": float(r["MaxNs"]) / 1e3})
    return out


def table(rows: List[Dict]) -> str:
    lines = ["| kernel | calls | total (us) | avg (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['name'][:60]} | {r['calls']} | {r['total_us']:.1f} | {r['avg_us']:.1f} | "
                     f"{r['min_us']:.1f} | {r['max_us']:.1f} |")
    return "\n".join(lines)


if __name__ == "__main__":
    p = sys.argv[1]
    rows = stats_from_db(p) if p.endswith(".db") else stats_from_csv(p)
    print(table(rows))
