"""Summaries of rocprofv3 result databases (SQLite ``*_results.db``) as short text.

    python -m tile_scheduled_persistent_amd.prof kernels DB [--cmd "..."]
        per-kernel calls, total / average / min / max duration (from --kernel-trace)
    python -m tile_scheduled_persistent_amd.prof counters DB --kernel NAME [--cmd "..."]
        per-dispatch counter values of one kernel (from --pmc runs), e.g. FETCH_SIZE / WRITE_SIZE
    python -m tile_scheduled_persistent_amd.prof traffic FETCH_DB WRITE_DB --calib-bytes B --read-bytes R --build-id ID [--cmd "..."]
        HBM bytes per launch of one kernel as JSON: FETCH_SIZE (KiB per dispatch) scaled by what
        the same counter reads for the library's stream-read kernel in the same run (each dispatch
        reads exactly R bytes with the decode kernel's own load form), WRITE_SIZE scaled by what it
        reads for the largest copy-kernel dispatch, a plain copy of B bytes (the stream read writes
        nothing); the copy-based FETCH factor is reported beside it as a cross-check

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


def _largest_copy(agg_by_kernel: dict) -> float:
    vals = [v for name, per in agg_by_kernel.items() if "copyBuffer" in name for v in per.values()]
    if not vals:
        raise SystemExit("no copy-kernel dispatch in the database: run with a calibration copy")
    return max(vals)


def _per_kernel(db: str, counter: str) -> dict:
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, value from counters_collection where counter_name = ?",
                       (counter,)).fetchall()
    out = {}
    for name, did, val in rows:
        out.setdefault(str(name), {}).setdefault(did, 0.0)
        out[str(name)][did] += float(val)
    return out


def _stream_read_kib(per: dict) -> list:
    return [v for name, d in per.items() if "stream_read" in name for v in d.values()]


def traffic(fetch_db: str, write_db: str, kernel: str, calib_bytes: int, read_bytes: int) -> dict:
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        per = _per_kernel(db, counter)
        copy_kib = _largest_copy(per)
        copy_factor = calib_bytes / (copy_kib * 1024.0)
        mine = [v for name, d in per.items() if kernel in name and "stream_read" not in name for v in d.values()]
        if not mine:
            raise SystemExit(f"no dispatch of {kernel} in {db}")
        rec = {"kib_per_dispatch": [round(v, 1) for v in mine], "mean_kib": statistics.mean(mine),
               "copy_kib": copy_kib, "copy_factor": copy_factor}
        factor = copy_factor
        if counter == "FETCH_SIZE":
            sr = _stream_read_kib(per)
            if not sr:
                raise SystemExit("no stream_read dispatch in the FETCH_SIZE database")
            rec["stream_read_kib"] = [round(v, 1) for v in sr]
            factor = read_bytes / (statistics.median(sr) * 1024.0)
            rec["stream_read_factor"] = factor
        rec["factor"] = factor
        rec["bytes_per_launch"] = statistics.mean(mine) * 1024.0 * factor
        res[counter] = rec
    res["traffic_bytes_per_launch"] = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["kernels", "counters", "traffic"])
    ap.add_argument("db")
    ap.add_argument("db2", nargs="?")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30)
    ap.add_argument("--read-bytes", type=int, default=2 << 30)
    ap.add_argument("--build-id", default="")
    ap.add_argument("--workload", default="")
    ap.add_argument("--kernel", default="tiles_worker")
    ap.add_argument("--cmd", default="")
    args = ap.parse_args(argv)
    if args.mode == "traffic":
        import json
        if not args.db2:
            raise SystemExit("traffic needs the FETCH_SIZE and the WRITE_SIZE database")
        d = traffic(args.db, args.db2, args.kernel, args.calib_bytes, args.read_bytes)
        d.update({"kernel": args.kernel, "workload": args.workload, "build_id": args.build_id,
                  "calibration": (f"FETCH_SIZE: median stream_read dispatch of the same run (each reads {args.read_bytes} "
                                  f"bytes with 16-byte non-temporal loads); WRITE_SIZE: largest __amd_rocclr_copyBuffer "
                                  f"dispatch of the same run, a copy of {args.calib_bytes} bytes"),
                  "command": args.cmd})
        print(json.dumps(d, indent=1))
        return 0
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
