"""Summarise rocprofv3 result databases (rocpd SQLite) as plain text.

    python -m clebsch_gordan_tensor_amd.profsum <results.db> [--match SUBSTR] [--pmc]

Prints, per kernel name (optionally filtered), the dispatch count, mean and
total duration, and with --pmc the mean of every collected counter per
dispatch. Used to produce the summaries committed under profiles/.
"""

import argparse
import sqlite3
import sys


def short(name, width=100):
    name = " ".join(name.split())
    return name if len(name) <= width else name[:width - 3] + "..."


def kernel_stats(cur, match):
    rows = cur.execute("select name, count(*), avg(duration), sum(duration) from kernels group by name "
                       "order by sum(duration) desc").fetchall()
    return [r for r in rows if match is None or match in r[0]]


def pmc_stats(cur, match):
    """Counter total per dispatch: all rows of a dispatch summed, divided by the
    number of distinct dispatches of that kernel."""
    q = ("select kernel_name, counter_name, sum(value) / count(distinct dispatch_id), "
         "count(distinct dispatch_id) from counters_collection "
         "group by kernel_name, counter_name order by kernel_name")
    try:
        rows = cur.execute(q).fetchall()
    except sqlite3.Error as e:
        print("no counter data: %s" % e)
        return []
    return [r for r in rows if match is None or match in r[0]]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--match", default=None)
    ap.add_argument("--pmc", action="store_true")
    a = ap.parse_args()
    cur = sqlite3.connect(a.db).cursor()
    print("%-100s %6s %14s %14s" % ("kernel", "calls", "mean_us", "total_ms"))
    for name, n, avg, tot in kernel_stats(cur, a.match):
        print("%-100s %6d %14.1f %14.3f" % (short(name), n, avg / 1e3, tot / 1e6))
    if a.pmc:
        rows = pmc_stats(cur, a.match)
        print()
        print("%-100s %-24s %18s %6s" % ("kernel", "counter", "per_dispatch", "n"))
        for name, ctr, val, n in rows:
            print("%-100s %-24s %18.1f %6d" % (short(name), ctr, val, n))
    return 0


if __name__ == "__main__":
    sys.exit(main())
