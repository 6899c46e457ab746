"""Summarise rocprofv3 output into short text tables.

  python rocprof_summary.py DIR            per-kernel calls, total and mean duration
                                           (from a --kernel-trace --stats run)
  python rocprof_summary.py --pmc DIR ...  per-kernel mean of each collected counter
                                           per dispatch (from --pmc runs)
  python rocprof_summary.py --counters DIR       per kernel: instructions per wave (VALU,
                                           MFMA, LDS), matrix-core and VALU busy shares
                                           (from one SQ counter pass; see counters())
  python rocprof_summary.py --stalls DIR         per kernel: shares of the waves' cycles
                                           issuing, waiting on dependencies and waiting
                                           for their turn (see stalls())
  python rocprof_summary.py --traffic FETCH_DIR WRITE_DIR KERNEL COPY_MIB SRC...
      HBM bytes per dispatch of the kernel whose name contains KERNEL, from a
      FETCH_SIZE run and a WRITE_SIZE run of the same command, each scaled by
      what the counter reads for the plain device copy of COPY_MIB MiB in that
      command; prints JSON with a hash of the source files SRC (the counters
      describe those sources only)

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
    name = name.replace("(anonymous namespace)::", "")
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


SIMDS = 1024  # 256 compute units x 4
XCDS = 8


def counters(path):
    """Per kernel, from a pass with SQ_WAVES, SQ_INSTS_VALU, SQ_INSTS_MFMA,
    SQ_INSTS_LDS, SQ_ACTIVE_INST_VALU, SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE: instructions per wave, and the shares of SIMD time the
    matrix cores and the vector ALU were busy.  GRBM_GUI_ACTIVE reads the
    sum over the XCDs of each one's active cycles, so one XCD's is the sum / 8.
    Matrix busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs) / (cycles x
    SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / (cycles x compute units), the
    vendor's VALUBusy formula.  The matrix share is read against the same
    counter on the matrix-core loop of libssd_peaks.so (the calibration line
    of each summary)."""
    out = {}
    for k, c in pmc_means(path).items():
        if "SQ_WAVES" not in c or "GRBM_GUI_ACTIVE" not in c:
            continue
        waves = c["SQ_WAVES"][0]
        cyc = c["GRBM_GUI_ACTIVE"][0] / XCDS
        row = {"dispatches": c["SQ_WAVES"][1], "waves": waves, "gui_cycles_per_xcd": cyc}
        for name in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS"):
            if name in c and waves:
                row[name.replace("SQ_INSTS_", "").lower() + "_per_wave"] = c[name][0] / waves
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and cyc:
            row["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"][0] / (cyc * SIMDS)
        if "SQ_ACTIVE_INST_VALU" in c and cyc:
            row["valu_busy"] = c["SQ_ACTIVE_INST_VALU"][0] / (cyc * SIMDS / 4)
        out[short(k)] = row
    return out


def stalls(path):
    """Per kernel, from a pass with SQ_WAVES, SQ_WAVE_CYCLES, SQ_WAIT_ANY,
    SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_ANY: the shares of the waves' cycles
    spent issuing instructions (ACTIVE_INST_ANY), waiting on their
    dependencies -- an s_waitcnt for loads or LDS reads, or a barrier --
    (WAIT_ANY), and ready but waiting for their turn to issue
    (WAIT_INST_ANY), each over SQ_WAVE_CYCLES."""
    out = {}
    for k, c in pmc_means(path).items():
        if "SQ_WAVE_CYCLES" not in c or not c["SQ_WAVE_CYCLES"][0]:
            continue
        wc = c["SQ_WAVE_CYCLES"][0]
        row = {"dispatches": c["SQ_WAVE_CYCLES"][1], "waves": c.get("SQ_WAVES", (0, 0))[0]}
        for name, key in (("SQ_ACTIVE_INST_ANY", "issue"), ("SQ_WAIT_ANY", "wait_dep"),
                          ("SQ_WAIT_INST_ANY", "wait_turn")):
            if name in c:
                row[key] = c[name][0] / wc
        out[short(k)] = row
    return out


def sources_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic(fetch_dir, write_dir, kernel, copy_mib, sources):
    f = pmc_means(fetch_dir)
    w = pmc_means(write_dir)
    copy_kib = copy_mib * 1024.0

    def pick(d, counter, sub):
        hits = [(k, v[counter]) for k, v in d.items() if sub in k and counter in v]
        if len(hits) != 1:
            raise SystemExit(f"{counter}: {len(hits)} kernels match {sub!r}: {[h[0] for h in hits]}")
        return hits[0]

    # the calibration copy: the largest dispatch of the streaming copy kernel
    # of libssd_peaks.so (bench.py --copy-mb COPY_MIB runs three of them)
    def copy_reading(path, counter):
        con = sqlite3.connect(_db(path))
        v = con.execute("select max(value) from counters_collection where counter_name = ? and "
                        "kernel_name like '%copy_kernel%'", (counter,)).fetchone()[0]
        if not v:
            raise SystemExit(f"{counter}: no copy kernel in the run")
        return float(v)

    fk, (fetch_kib, nf) = pick(f, "FETCH_SIZE", kernel)
    wk, (write_kib, nw) = pick(w, "WRITE_SIZE", kernel)
    ff = copy_kib / copy_reading(fetch_dir, "FETCH_SIZE")
    wf = copy_kib / copy_reading(write_dir, "WRITE_SIZE")
    return {
        "kernel": short(fk),
        "dispatches": [nf, nw],
        "fetch_kib_per_dispatch": fetch_kib,
        "write_kib_per_dispatch": write_kib,
        "fetch_factor": ff,
        "write_factor": wf,
        "bytes_per_dispatch": (fetch_kib * ff + write_kib * wf) * 1024.0,
        "copy_mib": copy_mib,
        "sources": [os.path.basename(p) for p in sources],
        "sources_sha256_16": sources_hash(sources),
    }


if __name__ == "__main__":
    if sys.argv[1] == "--traffic":
        import json
        fd, wd, kern, mib = sys.argv[2], sys.argv[3], sys.argv[4], float(sys.argv[5])
        print(json.dumps(traffic(fd, wd, kern, mib, sys.argv[6:]), indent=1))
    elif sys.argv[1] == "--counters":
        for k, r in sorted(counters(sys.argv[2]).items(), key=lambda kv: -kv[1]["waves"]):
            parts = [f"{k[:58]:58s} n={r['dispatches']:<4d}"]
            for name in ("valu_per_wave", "mfma_per_wave", "lds_per_wave"):
                if name in r:
                    parts.append(f"{name.split('_')[0]}/wave={r[name]:9.1f}")
            for name in ("mfma_busy", "valu_busy"):
                if name in r:
                    parts.append(f"{name}={100 * r[name]:5.1f}%")
            print("  ".join(parts))
    elif sys.argv[1] == "--stalls":
        for k, r in sorted(stalls(sys.argv[2]).items(), key=lambda kv: -kv[1]["waves"]):
            parts = [f"{k[:58]:58s} n={r['dispatches']:<4d} waves={r['waves']:<7.0f}"]
            for name in ("issue", "wait_dep", "wait_turn"):
                if name in r:
                    parts.append(f"{name}={100 * r[name]:5.1f}%")
            print("  ".join(parts))
    elif sys.argv[1] == "--pmc":
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
