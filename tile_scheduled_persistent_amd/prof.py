"""Summaries of rocprofv3 result databases (SQLite ``*_results.db``) as short text.

    python -m tile_scheduled_persistent_amd.prof kernels DB [--cmd "..."]
        per-kernel calls, total / average / min / max duration (from --kernel-trace)
    python -m tile_scheduled_persistent_amd.prof counters DB --kernel NAME [--cmd "..."]
        per-dispatch counter values of one kernel (from --pmc runs), e.g. FETCH_SIZE / WRITE_SIZE

The text goes to stdout; the command that produced the database is echoed in the header.
"""

from __future__ import annotations

import argparse
import sqlite3
import statistics
import sys


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    by = {}
    for name, dur in rows:
        by.setdefault(name, []).append(float(dur))
    out = []
    total = sum(sum(v) for v in by.values()) or 1.0
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append({"name": name, "calls": len(v), "total_ns": sum(v), "avg_ns": statistics.mean(v), "min_ns": min(v),
                    "max_ns": max(v), "pct": 100.0 * sum(v) / total})
    return out


def counter_values(db: str, kernel: str):
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info('counters_collection')")]
    rows = con.execute("select * from counters_collection").fetchall()
    recs = [dict(zip(cols, r)) for r in rows]
    name_key = "kernel_name" if "kernel_name" in cols else ("name" if "name" in cols else None)
    sel = [r for r in recs if name_key and kernel in str(r[name_key])]
    agg = {}
    for r in sel:
        cn = r.get("counter_name")
        val = r.get("value")
        did = r.get("dispatch_id")
        agg.setdefault(cn, {}).setdefault(did, 0.0)
        agg[cn][did] += float(val)
    return agg


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["kernels", "counters"])
    ap.add_argument("db")
    ap.add_argument("--kernel", default="tiles_worker")
    ap.add_argument("--cmd", default="")
    args = ap.parse_args(argv)
    if args.cmd:
        print(f"# command: {args.cmd}")
    if args.mode == "kernels":
        print(f"# rocprofv3 kernel trace summary of {args.db.split('/')[-1]}")
        print("# kernel | calls | total ms | avg us | min us | max us | % of GPU time")
        for r in kernel_stats(args.db):
            print(f"{r['name'][:100]} | {r['calls']} | {r['total_ns'] / 1e6:.3f} | {r['avg_ns'] / 1e3:.2f} | "
                  f"{r['min_ns'] / 1e3:.2f} | {r['max_ns'] / 1e3:.2f} | {r['pct']:.2f}")
    else:
        agg = counter_values(args.db, args.kernel)
        print(f"# rocprofv3 counters of kernels matching '{args.kernel}' in {args.db.split('/')[-1]}")
        for cn, per in agg.items():
            vals = list(per.values())
            print(f"{cn}: dispatches={len(vals)} mean={statistics.mean(vals):.1f} min={min(vals):.1f} max={max(vals):.1f}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
