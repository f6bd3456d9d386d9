"""Summaries of rocprofv3 output for the AReA kernels (tracing support).

    python -m resolution_diffusion_transformer_amd.profiling stats <kernel_stats.csv>
    python -m resolution_diffusion_transformer_amd.profiling counters <counter_collection.csv> [COUNTER]
    python -m resolution_diffusion_transformer_amd.profiling dispatches <kernel_trace.csv> NAME [NAME ...]

`stats` prints the per-kernel call count and average/total duration from
`rocprofv3 --kernel-trace --stats --output-format csv`.  `counters` prints,
per kernel, the dispatch count and the per-dispatch average of each counter
from `rocprofv3 --pmc ... --output-format csv` (counters reported per
hardware instance are summed within a dispatch first).  `dispatches` prints,
for each kernel whose name contains one of the NAMEs, the duration of every
dispatch in launch order (from `rocprofv3 --kernel-trace --output-format csv`).
"""
from __future__ import annotations

import collections
import csv
import sys


def short_name(name: str, width: int = 70) -> str:
    n = name.replace("area::(anonymous namespace)::", "")
    return n if len(n) <= width else n[:width - 3] + "..."


def kernel_stats(path: str, top: int = 20):
    rows = list(csv.DictReader(open(path)))
    key_dur = "TotalDurationNs" if "TotalDurationNs" in rows[0] else "Duration (Nsec)"
    out = []
    for r in rows:
        name = r.get("Name") or r.get("KERNEL_NAME") or ""
        calls = int(float(r.get("Calls", 0)))
        tot = float(r.get(key_dur, 0))
        avg = float(r.get("AverageNs", r.get("Average (Nsec)", tot / max(calls, 1))))
        out.append((name, calls, tot, avg))
    out.sort(key=lambda x: -x[2])
    return out[:top]


def format_stats(stats) -> str:
    lines = [f"{'kernel':72s} {'calls':>6s} {'total ms':>12s} {'avg ms':>10s}"]
    for name, calls, tot, avg in stats:
        lines.append(f"{short_name(name):72s} {calls:6d} {tot / 1e6:12.3f} {avg / 1e6:10.4f}")
    return "\n".join(lines)


def counters(path: str):
    """{kernel: {counter: [per-dispatch values]}}"""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(path)):
        disp = r.get("Dispatch_Id") or r.get("Correlation_Id")
        k = r["Kernel_Name"]
        per[(k, disp)][r["Counter_Name"]] += float(r["Counter_Value"])
        names[(k, disp)] = k
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for key, d in per.items():
        for c, v in d.items():
            out[names[key]][c].append(v)
    return out


def format_counters(cs, only=None) -> str:
    lines = []
    for k, d in sorted(cs.items(), key=lambda kv: -max(sum(v) for v in kv[1].values())):
        for c, vals in sorted(d.items()):
            if only and c != only:
                continue
            lines.append(f"{short_name(k):72s} {c:14s} dispatches {len(vals):5d} "
                         f"avg {sum(vals) / len(vals):16.1f} total {sum(vals):18.1f}")
    return "\n".join(lines)


def dispatches(path: str, names):
    """{kernel: [duration ns of each dispatch, in launch order]} for kernels
    whose name contains one of `names`."""
    rows = [r for r in csv.DictReader(open(path)) if any(n in r["Kernel_Name"] for n in names)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = collections.defaultdict(list)
    for r in rows:
        out[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def format_dispatches(ds) -> str:
    lines = []
    for k, durs in ds.items():
        lines.append(f"{short_name(k)}: {len(durs)} dispatches, us:")
        for i in range(0, len(durs), 10):
            lines.append("  " + " ".join(f"{d / 1e3:8.1f}" for d in durs[i:i + 10]))
    return "\n".join(lines)


def main(argv):
    if len(argv) < 2 or argv[0] not in ("stats", "counters", "dispatches"):
        print(__doc__)
        return 2
    if argv[0] == "stats":
        print(format_stats(kernel_stats(argv[1])))
    elif argv[0] == "dispatches":
        print(format_dispatches(dispatches(argv[1], argv[2:])))
    else:
        print(format_counters(counters(argv[1]), argv[2] if len(argv) > 2 else None))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
