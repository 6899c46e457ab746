"""The arithmetic of the profile summaries (rocprof_summary.py) on small
hand-made databases shaped like rocprofv3's SQLite output: the counter means
per dispatch, the busy and stall shares, and the traffic scaling by the
calibration copy."""
import os
import sqlite3

import pytest

import rocprof_summary as rs


def _db(tmp_path, name, rows, top=()):
    """A run directory holding one *_results.db with the counters table (and
    the top_kernels view's columns as a table)."""
    d = tmp_path / name
    os.makedirs(d / "node", exist_ok=True)
    con = sqlite3.connect(d / "node" / "run_results.db")
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, "
                "average real, percentage real)")
    con.executemany("insert into top_kernels values (?, ?, ?, ?, ?)", top)
    con.commit()
    con.close()
    return str(d)


K = "void ssd::demo_kernel<128>(float const*) [clone .kd]"


def test_means_and_busy_shares(tmp_path):
    # two dispatches; GRBM_GUI_ACTIVE sums the 8 XCDs' cycles
    rows = []
    for waves, valu, mfma_busy, active, gui in ((2048, 4.096e6, 4.0e9, 1.0e9, 8.0e7),
                                                (2048, 4.096e6, 6.0e9, 1.0e9, 8.0e7)):
        rows += [(K, "SQ_WAVES", waves), (K, "SQ_INSTS_VALU", valu),
                 (K, "SQ_VALU_MFMA_BUSY_CYCLES", mfma_busy),
                 (K, "SQ_ACTIVE_INST_VALU", active), (K, "GRBM_GUI_ACTIVE", gui)]
    r = rs.counters(_db(tmp_path, "sq", rows))["ssd::demo_kernel<128>"]
    assert r["dispatches"] == 2 and r["waves"] == 2048
    assert r["valu_per_wave"] == pytest.approx(2000.0)
    cyc = 8.0e7 / 8
    assert r["mfma_busy"] == pytest.approx(5.0e9 / (cyc * 1024))
    assert r["valu_busy"] == pytest.approx(1.0e9 / (cyc * 256))


def test_stall_shares(tmp_path):
    rows = [(K, "SQ_WAVES", 64), (K, "SQ_WAVE_CYCLES", 1000.0), (K, "SQ_ACTIVE_INST_ANY", 300.0),
            (K, "SQ_WAIT_ANY", 450.0), (K, "SQ_WAIT_INST_ANY", 250.0)]
    r = rs.stalls(_db(tmp_path, "st", rows))["ssd::demo_kernel<128>"]
    assert (r["issue"], r["wait_dep"], r["wait_turn"]) == pytest.approx((0.30, 0.45, 0.25))


def test_traffic_scaled_by_the_copy(tmp_path):
    copy = "void copy_kernel(float4 const*, float4*, long) [clone .kd]"
    mib = 256.0
    # the copy of 256 MiB reads as half its bytes fetched and all written
    fetch = _db(tmp_path, "f", [(copy, "FETCH_SIZE", mib * 1024 / 2), (copy, "FETCH_SIZE", 1.0),
                                (K, "FETCH_SIZE", 1000.0)])
    write = _db(tmp_path, "w", [(copy, "WRITE_SIZE", mib * 1024), (K, "WRITE_SIZE", 300.0)])
    src = tmp_path / "demo.hip"
    src.write_text("// demo\n")
    t = rs.traffic(fetch, write, "demo_kernel", mib, [str(src)])
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(1.0)
    assert t["bytes_per_dispatch"] == pytest.approx((1000.0 * 2.0 + 300.0) * 1024)
    assert t["sources"] == ["demo.hip"]
    assert t["sources_sha256_16"] == rs.sources_hash([str(src)])
    src.write_text("// changed\n")
    assert t["sources_sha256_16"] != rs.sources_hash([str(src)])


def test_kernel_stats_sorted_by_total(tmp_path):
    top = [("a_kernel", 10, 50.0, 5.0, 10.0), ("b_kernel", 2, 400.0, 200.0, 80.0)]
    rows = rs.kernel_stats(_db(tmp_path, "kt", [], top))
    assert [r[0] for r in rows] == ["b_kernel", "a_kernel"]
    assert rows[0][1:] == (2, 400.0, 200.0)
