"""Summarise rocprofv3 result databases (rocpd SQLite) and derive HBM traffic.

    python -m clebsch_gordan_tensor_amd.profsum <results.db> [--match SUBSTR] [--pmc] [--json OUT]
    python -m clebsch_gordan_tensor_amd.profsum --traffic OUT --fetch F.json --write W.json
           --calib-fetch CF.json --calib-write CW.json --calib-bytes B --units N --unit NAME
           --workload NAME --kernel BASE=src1,src2 [--kernel ...] [--per-call BASE=N ...]

The first form prints, per kernel name (optionally filtered), the dispatch
count, mean and total duration, and with --pmc the mean of every collected
counter per dispatch (all rows of a dispatch summed); --json also writes those
figures as JSON. The second form turns FETCH_SIZE / WRITE_SIZE summaries (KiB
per dispatch) into bytes per unit of work: each counter is scaled by what it
reads for a plain copy of known size (--calib-bytes read and written per
copy dispatch), and the dispatches of every instantiation of a kernel template
are added (one call of an operation launches each instantiation once, or N
times where --per-call BASE=N says so, e.g. one launch per output parity). The
entry (keyed kernel@workload) is tagged with a hash of the kernel's source
files, so a reader can tell when the counters no longer describe the code.
"""

import argparse
import hashlib
import json
import os
import sqlite3
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def short(name, width=100):
    name = " ".join(name.split())
    return name if len(name) <= width else name[:width - 3] + "..."


def source_hash(files):
    """First 16 hex digits of the SHA-256 of the named csrc files, in order."""
    h = hashlib.sha256()
    for n in files:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def base_name(full):
    """'void cgtp::conv_fwd_fused_kernel<float, ...>(...)' -> 'conv_fwd_fused_kernel'."""
    head = full.replace("(anonymous namespace)::", "").split("<")[0].split("(")[0]
    return head.split("::")[-1].split()[-1]


def summarise(a):
    cur = sqlite3.connect(a.db).cursor()
    out = {"kernels": {}, "counters": {}}
    print("%-100s %6s %14s %14s" % ("kernel", "calls", "mean_us", "total_ms"))
    for name, n, avg, tot in kernel_stats(cur, a.match):
        print("%-100s %6d %14.1f %14.3f" % (short(name), n, avg / 1e3, tot / 1e6))
        out["kernels"][name] = {"calls": n, "mean_us": avg / 1e3}
    if a.pmc:
        rows = pmc_stats(cur, a.match)
        print()
        print("%-100s %-24s %18s %6s" % ("kernel", "counter", "per_dispatch", "n"))
        for name, ctr, val, n in rows:
            print("%-100s %-24s %18.1f %6d" % (short(name), ctr, val, n))
            out["counters"].setdefault(name, {})[ctr] = {"per_dispatch": val, "n": n}
    if a.json:
        with open(a.json, "w") as f:
            json.dump(out, f, indent=1)
    return 0


def counter_by_base(path, counter):
    """{base kernel name: sum over its instantiations of the per-dispatch value}."""
    with open(path) as f:
        rec = json.load(f)["counters"]
    res = {}
    for name, ctrs in rec.items():
        if counter in ctrs:
            b = base_name(name)
            res[b] = res.get(b, 0.0) + ctrs[counter]["per_dispatch"]
    return res


def calib_factor(path, counter, known_bytes):
    """Bytes per counter unit, from the copy kernel (the largest reading in the file)."""
    with open(path) as f:
        rec = json.load(f)["counters"]
    vals = [c[counter]["per_dispatch"] for c in rec.values() if counter in c]
    return known_bytes / max(vals)


def traffic(a):
    ff = calib_factor(a.calib_fetch, "FETCH_SIZE", a.calib_bytes)
    wf = calib_factor(a.calib_write, "WRITE_SIZE", a.calib_bytes)
    fetch = counter_by_base(a.fetch, "FETCH_SIZE")
    write = counter_by_base(a.write, "WRITE_SIZE")
    per_call = {}
    for spec in a.per_call or []:
        base, n = spec.split("=")
        per_call[base] = int(n)
    rec = {}
    if os.path.exists(a.traffic):
        with open(a.traffic) as f:
            rec = json.load(f)
    rec["_note"] = ("HBM bytes per unit of work from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per "
                    "dispatch), each scaled by its reading for a plain copy of known size, summed over the "
                    "launches of one call (every instantiation of the kernel template)")
    for spec in a.kernel:
        base, srcs = spec.split("=")
        files = srcs.split(",")
        if base not in fetch or base not in write:
            print("%-28s no counter data, skipped" % base)
            continue
        n = per_call.get(base, 1)
        fb = n * fetch.get(base, 0.0) * ff / a.units
        wb = n * write.get(base, 0.0) * wf / a.units
        rec["%s@%s" % (base, a.workload)] = {"bytes_per_unit": round(fb + wb, 1), "fetch_bytes_per_unit": round(fb, 1),
                     "write_bytes_per_unit": round(wb, 1), "unit": a.unit, "workload": a.workload,
                     "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                     "sources": files, "source_hash": source_hash(files)}
        print("%-28s %12.1f B/%s (fetch %.1f, write %.1f)" % (base, fb + wb, a.unit, fb, wb))
    with open(a.traffic, "w") as f:
        json.dump(rec, f, indent=1)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db", nargs="?")
    ap.add_argument("--match", default=None)
    ap.add_argument("--pmc", action="store_true")
    ap.add_argument("--json", default=None)
    ap.add_argument("--traffic", default=None, help="traffic JSON to create or update")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--calib-bytes", type=float, help="bytes read (and written) per copy dispatch")
    ap.add_argument("--units", type=float, help="units of work per call (rows or edges)")
    ap.add_argument("--unit")
    ap.add_argument("--workload")
    ap.add_argument("--kernel", action="append", default=[], help="BASE=src1,src2 (csrc files)")
    ap.add_argument("--per-call", action="append", default=[], help="BASE=N dispatches of BASE per call (default 1)")
    a = ap.parse_args()
    if a.traffic:
        return traffic(a)
    if not a.db:
        ap.error("a results database is required")
    return summarise(a)


if __name__ == "__main__":
    sys.exit(main())
