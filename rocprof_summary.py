"""Summarise rocprofv3 output into short text tables.

  python rocprof_summary.py DIR            per-kernel calls, total and mean duration
                                           (from a --kernel-trace --stats run)
  python rocprof_summary.py --pmc DIR ...  per-kernel mean of each collected counter
                                           per dispatch (from --pmc runs)

DIR holds the run's ``*_results.db`` (rocprofv3's SQLite output).
"""
import glob
import os
import sqlite3
import sys
from collections import defaultdict


def _db(path):
    if os.path.isdir(path):
        dbs = sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))
        if not dbs:
            raise SystemExit(f"no *_results.db under {path}")
        return dbs[0]
    return path


def short(name):
    return name.split("(")[0].replace("void ", "")


def kernel_stats(path):
    """[(name, calls, total_us, mean_us)] sorted by total time."""
    con = sqlite3.connect(_db(path))
    rows = []
    # the top_kernels view reports durations in microseconds
    for name, calls, total, avg, _pct in con.execute(
            "select name, total_calls, total_duration, average, percentage from top_kernels"):
        rows.append((name, int(calls), float(total), float(avg)))
    rows.sort(key=lambda r: -r[2])
    return rows


def pmc_means(path):
    """{kernel: {counter: (mean per dispatch, dispatches)}}"""
    con = sqlite3.connect(_db(path))
    acc = defaultdict(lambda: defaultdict(list))
    for kname, counter, value in con.execute(
            "select kernel_name, counter_name, value from counters_collection"):
        acc[kname][counter].append(float(value))
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in d.items()} for k, d in acc.items()}


if __name__ == "__main__":
    if sys.argv[1] == "--pmc":
        merged = defaultdict(dict)
        for d in sys.argv[2:]:
            for k, cs in pmc_means(d).items():
                merged[k].update(cs)
        for k in sorted(merged):
            items = "  ".join(f"{c}={m:.6g} (n={n})" for c, (m, n) in sorted(merged[k].items()))
            print(f"{short(k)[:60]:60s} {items}")
    else:
        for name, calls, total, mean in kernel_stats(sys.argv[1]):
            print(f"{short(name)[:70]:70s} calls={calls:6d} total_us={total:11.1f} "
                  f"mean_us={mean:9.2f}")
