"""Text summaries of rocprofv3 output (the SQLite database it writes).

    python -m harness.rocprof_summary kernels DIR [--top N]
    python -m harness.rocprof_summary counters DIR [--kernel SUBSTR] [--dispatches]

`kernels` prints, per kernel name, the number of dispatches and the average,
median, minimum, maximum and total duration (from a --kernel-trace run); `counters`
prints, per kernel and counter, the mean value per dispatch (from a --pmc
run), and with --dispatches every dispatch's value in dispatch order (to tell
apart launches of one kernel with different sizes, such as the copies of a
calibration run).  DIR is the directory given to rocprofv3 with -d; every *.db below it is
read.
"""
from __future__ import annotations

import argparse
import collections
import glob
import os
import sqlite3
import sys


def _dbs(d: str) -> list[str]:
    paths = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not paths:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return paths


def _median(v: list[float]) -> float:
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def kernel_stats(d: str) -> list[tuple[str, int, float, float, float, float, float]]:
    """(name, calls, avg_us, median_us, min_us, max_us, total_us), largest total first."""
    acc: dict[str, list[float]] = collections.defaultdict(list)
    for path in _dbs(d):
        con = sqlite3.connect(path)
        for name, dur in con.execute("select name, end - start from kernels"):
            acc[name].append(dur / 1000.0)
        con.close()
    rows = [(n, len(v), sum(v) / len(v), _median(v), min(v), max(v), sum(v)) for n, v in acc.items()]
    rows.sort(key=lambda r: -r[6])
    return rows


def counter_means(d: str, kernel_substr: str = "") -> dict[str, dict[str, tuple[float, int]]]:
    """{kernel: {counter: (mean value per dispatch, dispatches)}}."""
    sums: dict[tuple[str, str], list[float]] = collections.defaultdict(list)
    for path in _dbs(d):
        con = sqlite3.connect(path)
        q = ("select kernel_name, counter_name, dispatch_id, sum(value) from counters_collection "
             "where kernel_name like ? group by kernel_name, counter_name, dispatch_id")
        for k, c, _, v in con.execute(q, (f"%{kernel_substr}%",)):
            sums[(k, c)].append(float(v))
        con.close()
    out: dict[str, dict[str, tuple[float, int]]] = collections.defaultdict(dict)
    for (k, c), v in sums.items():
        out[k][c] = (sum(v) / len(v), len(v))
    return out


def counter_dispatches(d: str, kernel_substr: str = "") -> list[tuple[str, str, int, float]]:
    """(kernel, counter, dispatch id, value summed over instances), in dispatch order."""
    rows = []
    for path in _dbs(d):
        con = sqlite3.connect(path)
        q = ("select kernel_name, counter_name, dispatch_id, sum(value) from counters_collection "
             "where kernel_name like ? group by kernel_name, counter_name, dispatch_id order by dispatch_id")
        rows += [(k, c, int(i), float(v)) for k, c, i, v in con.execute(q, (f"%{kernel_substr}%",))]
        con.close()
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["kernels", "counters"])
    ap.add_argument("dir")
    ap.add_argument("--top", type=int, default=12)
    ap.add_argument("--kernel", default="")
    ap.add_argument("--dispatches", action="store_true")
    a = ap.parse_args(argv)
    if a.what == "kernels":
        print(f"{'calls':>6} {'avg_us':>9} {'med_us':>9} {'min_us':>9} {'max_us':>9} {'total_us':>11}  kernel")
        for n, c, avg, med, mn, mx, tot in kernel_stats(a.dir)[: a.top]:
            print(f"{c:6d} {avg:9.2f} {med:9.2f} {mn:9.2f} {mx:9.2f} {tot:11.1f}  {n}")
    elif a.dispatches:
        for k, c, i, v in counter_dispatches(a.dir, a.kernel):
            print(f"{i:8d} {c:16s} {v:16.1f}  {k}")
    else:
        for k, cs in counter_means(a.dir, a.kernel).items():
            print(k)
            for c, (v, n) in sorted(cs.items()):
                print(f"    {c:24s} {v:18.1f}  (dispatches: {n})")
    return 0


if __name__ == "__main__":
    sys.exit(main())
