"""Reduce rocprofv3 CSV output to short per-kernel text summaries.

    python3 profsum.py stats  <kernel_stats.csv>  [--match REGEX]
    python3 profsum.py counters <counter_collection.csv> [--match REGEX]
        [--delete]
    python3 profsum.py traffic --fetch F.csv --write W.csv --match REGEX
        --copy-match REGEX --copy-bytes N --source FILE [FILE ...] [--delete]

`stats` lists calls and average / min / max duration per kernel (from
`rocprofv3 --kernel-trace --stats --output-format csv`). `counters` sums the
rows of each dispatch per counter (a counter can be reported per hardware
instance) and prints, per kernel and counter, the number of dispatches and
the mean, min and max of the per-dispatch totals (from `rocprofv3 --pmc ...
--output-format csv`). With --delete the counter CSV is removed after it has
been read, so large raw files need not leave the machine that wrote them.

`traffic` turns one FETCH_SIZE pass and one WRITE_SIZE pass (KiB per
dispatch) into HBM bytes per call of the kernels matched by --match (one call
= one dispatch of each): each counter is scaled by the ratio of a known copy's
size (--copy-bytes, the largest dispatch of the --copy-match kernel) to what
the same counter reads for that copy. It also prints the sha256 of the given
kernel sources, so a reader can tell whether the figure still describes the
code.
"""
import hashlib
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


def _per_dispatch(path, rx):
    per = defaultdict(float)
    names = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name", "")
            if not rx.search(name):
                continue
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = name
    return per, names


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic(fetch, write, match, copy_match, copy_bytes, sources):
    rx, crx = re.compile(match), re.compile(copy_match)
    lines = []
    total = 0.0
    for label, path in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        cper, _ = _per_dispatch(path, crx)
        copy_kib = max(cper.values())
        factor = copy_bytes / (copy_kib * 1024.0)
        lines.append(f"{label} calibration: copy of {copy_bytes} bytes reads {copy_kib:.1f} KiB -> factor {factor:.4f}")
        per, names = _per_dispatch(path, rx)
        byk = defaultdict(list)
        for d, v in per.items():
            byk[names[d]].append(v)
        for name, vs in sorted(byk.items()):
            mean = sum(vs) / len(vs)
            b = mean * 1024.0 * factor
            total += b
            lines.append(f"  {label} {len(vs):5d} dispatches, mean {mean:.1f} KiB -> {b / 1e6:.3f} MB per call  {_short(name)}")
    lines.append(f"traffic_bytes_per_call: {total:.0f}")
    lines.append(f"sources: {' '.join(sources)}")
    lines.append(f"source_sha256: {source_hash(sources)}")
    return "\n".join(lines)


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("kind", choices=["stats", "counters", "traffic"])
    p.add_argument("path", nargs="?")
    p.add_argument("--match", default=None)
    p.add_argument("--delete", action="store_true")
    p.add_argument("--fetch")
    p.add_argument("--write")
    p.add_argument("--copy-match", default=r"copyBuffer|copy_kernel")
    p.add_argument("--copy-bytes", type=int, default=0)
    p.add_argument("--source", nargs="*", default=[])
    a = p.parse_args(argv)
    if a.kind == "traffic":
        print(traffic(a.fetch, a.write, a.match, a.copy_match, a.copy_bytes, a.source))
        if a.delete:
            os.remove(a.fetch)
            os.remove(a.write)
        return 0
    text = stats(a.path, a.match) if a.kind == "stats" else counters(a.path, a.match)
    print(text)
    if a.delete:
        os.remove(a.path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
