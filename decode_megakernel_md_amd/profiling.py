"""Profiling helpers: summarise rocprofv3 output.

    python -m decode_megakernel_md_amd.profiling <kernel_stats.csv | results.db>
    python -m decode_megakernel_md_amd.profiling gaps <kernel_trace.csv | results.db> [kernel-name-substring]
    python -m decode_megakernel_md_amd.profiling pmc <counter_collection.csv>
    python -m decode_megakernel_md_amd.profiling traffic <fetch.csv> <write.csv> [workload] [batch]

The first form prints a per-kernel table (calls, total/avg/min/max duration
in microseconds) from rocprofv3's --stats CSV or its rocpd SQLite database.
The second lists, per run of back-to-back dispatches of the named kernel
(default md_megakernel, which also serves the multi-launch baseline's
per-phase launches), the busy time and the idle time between consecutive
dispatches: the bubbles a single persistent launch removes.  The third averages each
counter per dispatch and kernel from a --pmc run.  The fourth turns a
FETCH_SIZE run and a WRITE_SIZE run of profile_run.py (a 1 GiB device copy,
then decode steps) into HBM bytes per megakernel launch, each counter scaled
by what it reads for the copy, and records them in traffic.json together
with a hash of the kernel sources they were measured on (bench.py reports
them only while the sources still hash the same)."""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sqlite3
import sys
from typing import Dict, List

HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(HERE, "traffic.json")
KERNEL_SOURCES = ("md_kernel.hip", "md_device.h", "md_model.h")
COPY_BYTES = 1 << 30       # profile_run.py's calibration copy
COPY_KERNEL = "copyBuffer"


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


def dispatches(path: str, needle: str) -> List[tuple]:
    """(start_ns, end_ns) of every dispatch whose kernel name contains needle, by start time."""
    if path.endswith(".db"):
        db = sqlite3.connect(path)
        rows = db.execute("select name, start, end from kernels order by start").fetchall()
        return [(int(r[1]), int(r[2])) for r in rows if needle in r[0]]
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if needle in r["Kernel_Name"]:
                out.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out.sort()
    return out


def gaps(d: List[tuple], break_ns: int = 1_000_000) -> Dict:
    """Idle time between consecutive dispatches; a gap longer than break_ns is
    taken as the host pausing between runs and starts a new run."""
    runs, cur = [], [d[0]] if d else []
    for a, b in zip(d, d[1:]):
        if b[0] - a[1] > break_ns:
            runs.append(cur)
            cur = [b]
        else:
            cur.append(b)
    if cur:
        runs.append(cur)
    busy = sum(e - s for r in runs for s, e in r)
    span = sum(r[-1][1] - r[0][0] for r in runs)
    g = [b[0] - a[1] for r in runs for a, b in zip(r, r[1:])]
    return {"dispatches": len(d), "runs": len(runs), "busy_us": busy / 1e3, "span_us": span / 1e3,
            "idle_us": (span - busy) / 1e3, "gaps": len(g), "mean_gap_us": (sum(g) / len(g) / 1e3) if g else 0.0,
            "max_gap_us": (max(g) / 1e3) if g else 0.0}


def pmc(path: str) -> List[Dict]:
    """Per (kernel, counter): dispatches and the mean counter value per dispatch."""
    acc: Dict[tuple, List[float]] = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            acc.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return [{"kernel": k[0], "counter": k[1], "dispatches": len(v), "mean": sum(v) / len(v), "min": min(v),
             "max": max(v)} for k, v in sorted(acc.items(), key=lambda kv: -sum(kv[1]))]


def kernel_source_hash() -> str:
    """SHA-256 over the device sources of the megakernel."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_record(fetch_csv: str, write_csv: str, workload: str, batch: int) -> Dict:
    """HBM bytes per megakernel launch (either build) from a FETCH_SIZE and a WRITE_SIZE
    run.  Both counters are in KiB per dispatch; the calibration copy of
    COPY_BYTES read and written gives each counter's bytes-per-unit factor."""
    out = {"workload": workload, "batch": batch, "kernel_sha256": kernel_source_hash()}
    for name, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = list(csv.DictReader(open(path)))
        copy = sum(float(r["Counter_Value"]) for r in rows if COPY_KERNEL in r["Kernel_Name"])
        mk = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] in ("md_megakernel", "md_megakernel_w64")]
        if copy <= 0 or not mk:
            raise ValueError(f"{path}: no calibration copy or no megakernel dispatch")
        factor = COPY_BYTES / (copy * 1024.0)
        out[name + "_kib_per_dispatch"] = sum(mk) / len(mk)
        out[name + "_factor"] = factor
        out[name + "_bytes"] = sum(mk) / len(mk) * 1024.0 * factor
    out["bytes"] = out["fetch_bytes"] + out["write_bytes"]
    return out


def _traffic_records() -> List[Dict]:
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return []
    return rec.get("records", []) if isinstance(rec, dict) and "records" in rec else ([rec] if rec else [])


def store_traffic(rec: Dict) -> None:
    """Keep rec in traffic.json, replacing any record of its workload and batch."""
    recs = [r for r in _traffic_records() if (r.get("workload"), r.get("batch")) != (rec["workload"], rec["batch"])]
    recs.append(rec)
    recs.sort(key=lambda r: (r["workload"], r["batch"]))
    with open(TRAFFIC_JSON, "w") as f:
        json.dump({"records": recs}, f, indent=1)


def traffic_for(workload: str, batch: int):
    """The recorded HBM bytes per launch for this workload and batch, or None
    when there is no record or the kernel sources changed since."""
    h = kernel_source_hash()
    for rec in _traffic_records():
        if rec.get("workload") == workload and rec.get("batch") == batch and rec.get("kernel_sha256") == h:
            return rec
    return None


if __name__ == "__main__":
    if sys.argv[1] == "pmc":
        print("| kernel | counter | dispatches | mean per dispatch | min | max |")
        print("|---|---|---|---|---|---|")
        for r in pmc(sys.argv[2]):
            print(f"| {r['kernel'][:70]} | {r['counter']} | {r['dispatches']} | {r['mean']:.1f} | {r['min']:.1f} | "
                  f"{r['max']:.1f} |")
    elif sys.argv[1] == "traffic":
        wl = sys.argv[4] if len(sys.argv) > 4 else "dense_27b"
        b = int(sys.argv[5]) if len(sys.argv) > 5 else 1
        rec = traffic_record(sys.argv[2], sys.argv[3], wl, b)
        store_traffic(rec)
        print(json.dumps(rec, indent=1))
    elif sys.argv[1] == "gaps":
        needle = sys.argv[3] if len(sys.argv) > 3 else "md_megakernel"
        d = dispatches(sys.argv[2], needle)
        print("| run | dispatches | busy (us) | span (us) | idle between dispatches (us) | gaps | "
              "mean gap (us) | max gap (us) |")
        print("|---|---|---|---|---|---|---|---|")
        # one row per run (dispatches separated by less than 1 ms), then all of them
        runs, cur = [], d[:1]
        for a, b in zip(d, d[1:]):
            if b[0] - a[1] > 1_000_000:
                runs.append(cur)
                cur = [b]
            else:
                cur.append(b)
        if cur:
            runs.append(cur)
        for i, run in enumerate(runs + [d]):
            r = gaps(run)
            name = f"{i + 1}" if i < len(runs) else "all"
            print(f"| {name} | {r['dispatches']} | {r['busy_us']:.1f} | {r['span_us']:.1f} | "
                  f"{r['idle_us']:.1f} | {r['gaps']} | {r['mean_gap_us']:.2f} | {r['max_gap_us']:.2f} |")
    else:
        p = sys.argv[1]
        rows = stats_from_db(p) if p.endswith(".db") else stats_from_csv(p)
        print(table(rows))
