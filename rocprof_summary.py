"""Summarise a rocprofv3 run (its SQLite ``*_results.db`` or ``kernel_stats.csv``)
into a short per-kernel text table: calls, total and mean duration."""
import csv
import glob
import os
import sqlite3
import sys


def kernel_stats(path):
    """[(name, calls, total_us, mean_us)] sorted by total time."""
    rows = []
    dbs = glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True) if os.path.isdir(path) else [path]
    csvs = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True) if os.path.isdir(path) else []
    if dbs and dbs[0].endswith(".db"):
        con = sqlite3.connect(dbs[0])
        for name, calls, total, avg, _pct in con.execute(
                "select name, total_calls, total_duration, average, percentage from top_kernels"):
            # the top_kernels view reports durations in microseconds
            rows.append((name, int(calls), float(total), float(avg)))
    elif csvs:
        with open(csvs[0]) as f:
            for r in csv.DictReader(f):
                rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                             float(r["AverageNs"]) / 1e3))
    rows.sort(key=lambda r: -r[2])
    return rows


def short(name):
    return name.split("(")[0].replace("void ", "")


if __name__ == "__main__":
    for name, calls, total, mean in kernel_stats(sys.argv[1]):
        print(f"{short(name)[:70]:70s} calls={calls:6d} total_us={total:11.1f} mean_us={mean:9.2f}")
