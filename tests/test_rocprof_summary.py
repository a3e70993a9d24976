"""The rocprofv3 summary tool on a hand-made database (no GPU): per-kernel
call counts and mean / median / min / max / total durations, the counter
means per dispatch, and the printed table."""
import os
import sqlite3
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from harness import rocprof_summary as rs  # noqa: E402


def _db(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    con = sqlite3.connect(str(d / "run_results.db"))
    con.execute("create table kernels (name text, start integer, end integer)")
    # durations in ns: gemm 10, 20, 30, 100 us; combine 5, 7 us
    rows = [("gemm", 0, 10_000), ("gemm", 50_000, 70_000), ("gemm", 100_000, 130_000),
            ("gemm", 200_000, 300_000), ("combine", 0, 5_000), ("combine", 10_000, 17_000)]
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.execute("create table counters_collection (kernel_name text, counter_name text, dispatch_id integer, "
                "value real)")
    # two dispatches of gemm; the counter arrives split over two instances in the first
    cnt = [("gemm", "FETCH_SIZE", 1, 100.0), ("gemm", "FETCH_SIZE", 1, 50.0), ("gemm", "FETCH_SIZE", 2, 250.0),
           ("combine", "FETCH_SIZE", 3, 8.0)]
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", cnt)
    con.commit()
    con.close()
    return str(d)


def test_kernel_stats(tmp_path):
    d = _db(tmp_path)
    stats = {r[0]: r[1:] for r in rs.kernel_stats(d)}
    calls, avg, med, mn, mx, tot = stats["gemm"]
    assert calls == 4 and avg == 40.0 and med == 25.0 and mn == 10.0 and mx == 100.0 and tot == 160.0
    calls, avg, med, mn, mx, tot = stats["combine"]
    assert calls == 2 and avg == 6.0 and med == 6.0 and mn == 5.0 and mx == 7.0 and tot == 12.0
    # largest total first
    assert [r[0] for r in rs.kernel_stats(d)] == ["gemm", "combine"]


def test_counter_means(tmp_path):
    d = _db(tmp_path)
    m = rs.counter_means(d, "gemm")
    assert set(m) == {"gemm"}
    mean, n = m["gemm"]["FETCH_SIZE"]
    assert n == 2 and mean == 200.0          # (100 + 50 + 250) / 2 dispatches
    disp = rs.counter_dispatches(d)
    assert [(k, i, v) for k, _, i, v in disp] == [("gemm", 1, 150.0), ("gemm", 2, 250.0), ("combine", 3, 8.0)]


def test_printed_table(tmp_path):
    d = _db(tmp_path)
    r = subprocess.run([sys.executable, "-m", "harness.rocprof_summary", "kernels", d], capture_output=True,
                       text=True, cwd=ROOT, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.splitlines()
    assert lines[0].split() == ["calls", "avg_us", "med_us", "min_us", "max_us", "total_us", "kernel"]
    assert lines[1].split() == ["4", "40.00", "25.00", "10.00", "100.00", "160.0", "gemm"]
