"""Reduce rocprofv3 CSV output to short per-kernel text summaries.

    python -m tiered_quantized_kv_amd.profsum stats  <kernel_stats.csv>  [--match REGEX]
    python -m tiered_quantized_kv_amd.profsum counters <counter_collection.csv> [--match REGEX]
        [--delete]

`stats` lists calls and average / min / max duration per kernel (from
`rocprofv3 --kernel-trace --stats --output-format csv`). `counters` sums the
rows of each dispatch per counter (a counter can be reported per hardware
instance) and prints, per kernel and counter, the number of dispatches and
the mean, min and max of the per-dispatch totals (from `rocprofv3 --pmc ...
--output-format csv`). With --delete the counter CSV is removed after it has
been read, so large raw files need not leave the machine that wrote them.
"""
import argparse
import csv
import os
import re
import sys
from collections import defaultdict


def _short(name, width=90):
    name = re.sub(r"\s+", " ", name)
    return name if len(name) <= width else name[: width - 3] + "..."


def stats(path, match):
    rx = re.compile(match) if match else None
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if rx and not rx.search(r["Name"]):
                continue
            rows.append(r)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10}  kernel"]
    for r in rows:
        out.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                   f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['TotalDurationNs']) / 1e6:10.3f}  {_short(r['Name'])}")
    return "\n".join(out)


def counters(path, match):
    rx = re.compile(match) if match else None
    per = defaultdict(float)            # (kernel, counter, dispatch) -> total
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name", "")
            if rx and not rx.search(name):
                continue
            per[(name, r["Counter_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
    agg = defaultdict(list)
    for (name, ctr, _), v in per.items():
        agg[(name, ctr)].append(v)
    out = [f"{'dispatches':>10} {'mean':>16} {'min':>16} {'max':>16}  counter  kernel"]
    for (name, ctr), vs in sorted(agg.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        out.append(f"{len(vs):10d} {sum(vs) / len(vs):16.1f} {min(vs):16.1f} {max(vs):16.1f}  {ctr}  {_short(name)}")
    return "\n".join(out)


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("kind", choices=["stats", "counters"])
    p.add_argument("path")
    p.add_argument("--match", default=None)
    p.add_argument("--delete", action="store_true")
    a = p.parse_args(argv)
    text = stats(a.path, a.match) if a.kind == "stats" else counters(a.path, a.match)
    print(text)
    if a.delete:
        os.remove(a.path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
