"""rocprofv3 harness: turn kernel traces and PMC counters into the numbers the
benchmark reports (per-kernel average duration, achieved GB/s or TFLOPS,
HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE).

Typical use on an MI355X host:

  rocprofv3 --kernel-trace --stats -f csv -d OUT -o run -- python bench.py
  python -m quantized_gemm_groupwise_amd.rocprof stats OUT --match gemv_kernel

  rocprofv3 --pmc FETCH_SIZE -f csv -d OUT_F -o run -- python bench.py ...
  rocprofv3 --pmc WRITE_SIZE -f csv -d OUT_W -o run -- python bench.py ...
  python -m quantized_gemm_groupwise_amd.rocprof pmc OUT_F OUT_W --match gemv_kernel

Counter passes are kept separate (one counter block per run), as the
counters of one pass must fit the hardware in a single collection.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# sources whose text decides the decode GEMV kernel (its counters go stale
# when any of them changes)
GEMV_SOURCES = ("gemv_group.hip", "gemv_core.h", "gq_internal.h", "gq_device.h")


def source_digest(names=GEMV_SOURCES) -> str:
    """First 16 hex digits of the SHA-256 of the named csrc files, in order."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(dirpath: str, suffix: str) -> list:
    return sorted(glob.glob(os.path.join(dirpath, "**", f"*{suffix}"), recursive=True))


def read_csv(path: str) -> list:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_trace(dirpath: str) -> list:
    """Per-dispatch rows: name, duration_ns, grid, workgroup."""
    rows = []
    for p in _find(dirpath, "kernel_trace.csv"):
        for r in read_csv(p):
            name = r.get("Kernel_Name") or r.get("KernelName") or ""
            try:
                start = int(r.get("Start_Timestamp") or r.get("BeginNs"))
                end = int(r.get("End_Timestamp") or r.get("EndNs"))
            except (TypeError, ValueError):
                continue
            grid = tuple(int(r.get(k, 0) or 0) for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
            wg = tuple(int(r.get(k, 0) or 0) for k in ("Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"))
            rows.append({"name": name, "start": start, "duration_ns": end - start, "grid": grid,
                         "workgroup": wg, "dispatch": int(r.get("Dispatch_Id", 0) or 0)})
    rows.sort(key=lambda r: r["start"])
    return rows


def kernel_stats(dirpath: str) -> list:
    out = []
    for p in _find(dirpath, "kernel_stats.csv"):
        for r in read_csv(p):
            out.append({"name": r.get("Name", ""), "calls": int(r.get("Calls", 0) or 0),
                        "total_ns": float(r.get("TotalDurationNs", 0) or 0),
                        "avg_ns": float(r.get("AverageNs", 0) or 0),
                        "min_ns": float(r.get("MinNs", 0) or 0), "max_ns": float(r.get("MaxNs", 0) or 0),
                        "pct": float(r.get("Percentage", 0) or 0)})
    return out


def select(rows: list, match: str, grid=None) -> list:
    rx = re.compile(match)
    return [r for r in rows if rx.search(r["name"]) and (grid is None or r["grid"] == tuple(grid))]


def summarize_dispatches(rows: list) -> dict:
    d = [r["duration_ns"] for r in rows]
    if not d:
        return {"dispatches": 0}
    return {"dispatches": len(d), "avg_us": statistics.fmean(d) / 1e3,
            "median_us": statistics.median(d) / 1e3, "min_us": min(d) / 1e3, "max_us": max(d) / 1e3}


def pmc_values(dirpath: str, counter: str, match: str, grid=None, first=None) -> list:
    """Per-dispatch values of one counter for kernels matching `match` (and
    launched with `grid` work-items, if given), in dispatch order; `first`
    keeps only the first that many dispatches."""
    rx = re.compile(match)
    vals = {}
    for p in _find(dirpath, "counter_collection.csv"):
        for r in read_csv(p):
            if (r.get("Counter_Name") or "") != counter:
                continue
            if not rx.search(r.get("Kernel_Name", "")):
                continue
            if grid is not None and int(r.get("Grid_Size", 0) or 0) != grid:
                continue
            key = (p, int(r.get("Dispatch_Id", 0) or 0))
            vals[key] = vals.get(key, 0.0) + float(r.get("Counter_Value", 0) or 0)
    out = [v for _, v in sorted(vals.items())]
    return out[:first] if first else out


def _main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m quantized_gemm_groupwise_amd.rocprof")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats", help="kernel durations from a --kernel-trace --stats run")
    s.add_argument("dir")
    s.add_argument("--match", default=".")
    s.add_argument("--grid", default=None, help="x,y,z grid (work-items) to select one launch shape")
    s.add_argument("--bytes", type=float, default=None, help="algorithmic bytes per dispatch")
    s.add_argument("--flops", type=float, default=None, help="algorithmic flops per dispatch")
    s.add_argument("--top", type=int, default=12)
    q = sub.add_parser("pmc", help="FETCH_SIZE / WRITE_SIZE per dispatch")
    q.add_argument("fetch_dir")
    q.add_argument("write_dir")
    q.add_argument("--match", required=True)
    q.add_argument("--grid", type=int, default=None, help="total work-items of the selected launches")
    q.add_argument("--calib-match", default=None, help="copy kernel regex for calibration")
    q.add_argument("--calib-first", type=int, default=None,
                   help="use only the first N matching copy dispatches (the calibration copies)")
    q.add_argument("--calib-bytes", type=float, default=None, help="bytes the copy kernel moves each way")
    q.add_argument("--json", default=None, help="write the calibrated numbers to this file")
    q.add_argument("--kernel-desc", default="", help="description of the kernel and shape (json)")
    q.add_argument("--algo-bytes", type=float, default=None, help="algorithmic bytes per dispatch (json)")
    q.add_argument("--command", action="append", default=[], help="profiling command (json, repeatable)")
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        st = sorted(kernel_stats(a.dir), key=lambda r: -r["total_ns"])
        print(f"{'kernel':90s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'%':>6s}")
        for r in st[: a.top]:
            print(f"{r['name'][:90]:90s} {r['calls']:7d} {r['avg_ns'] / 1e3:9.2f} {r['min_ns'] / 1e3:9.2f} "
                  f"{r['max_ns'] / 1e3:9.2f} {r['pct']:6.2f}")
        grid = tuple(int(v) for v in a.grid.split(",")) if a.grid else None
        rows = select(kernel_trace(a.dir), a.match, grid)
        sm = summarize_dispatches(rows)
        print(f"\nselected dispatches (match={a.match!r}, grid={grid}): {sm}")
        if sm.get("dispatches"):
            if a.bytes:
                print(f"achieved: {a.bytes / (sm['avg_us'] * 1e-6) / 1e9:.1f} GB/s at the average duration")
            if a.flops:
                print(f"achieved: {a.flops / (sm['avg_us'] * 1e-6) / 1e12:.1f} TFLOP/s at the average duration")
    else:
        f = pmc_values(a.fetch_dir, "FETCH_SIZE", a.match, a.grid)
        w = pmc_values(a.write_dir, "WRITE_SIZE", a.match, a.grid)
        print(f"FETCH_SIZE KiB per dispatch: n={len(f)} mean={statistics.fmean(f) if f else 0:.1f}")
        print(f"WRITE_SIZE KiB per dispatch: n={len(w)} mean={statistics.fmean(w) if w else 0:.1f}")
        if a.calib_match and a.calib_bytes:
            cf = pmc_values(a.fetch_dir, "FETCH_SIZE", a.calib_match, first=a.calib_first)
            cw = pmc_values(a.write_dir, "WRITE_SIZE", a.calib_match, first=a.calib_first)
            if cf and cw:
                kf = a.calib_bytes / (statistics.fmean(cf) * 1024)
                kw = a.calib_bytes / (statistics.fmean(cw) * 1024)
                print(f"copy calibration: bytes per reported byte fetch={kf:.4f} write={kw:.4f}")
                if f and w:
                    tb = statistics.fmean(f) * 1024 * kf + statistics.fmean(w) * 1024 * kw
                    print(f"calibrated HBM traffic per dispatch: {tb:.0f} bytes")
                    if a.json:
                        out = {
                            "kernel": a.kernel_desc,
                            "source_digest": source_digest(),
                            "source_files": [f"quantized_gemm_groupwise_amd/csrc/{n}" for n in GEMV_SOURCES],
                            "dispatches_fetch": len(f), "dispatches_write": len(w),
                            "fetch_size_kib_per_dispatch": round(statistics.fmean(f), 1),
                            "write_size_kib_per_dispatch": round(statistics.fmean(w), 1),
                            "calibration": {
                                "kernel": "hipMemcpy device-to-device (__amd_rocclr_copyBuffer) of 256 MiB",
                                "bytes_each_way": int(a.calib_bytes),
                                "fetch_size_kib": round(statistics.fmean(cf), 1),
                                "write_size_kib": round(statistics.fmean(cw), 1),
                                "fetch_factor": round(kf, 5), "write_factor": round(kw, 5)},
                            "traffic_bytes_per_launch": int(round(tb)),
                            "algorithmic_bytes_per_launch": int(a.algo_bytes) if a.algo_bytes else None,
                            "traffic_over_algorithmic": round(tb / a.algo_bytes, 4) if a.algo_bytes else None,
                            "commands": a.command,
                        }
                        with open(a.json, "w") as fo:
                            json.dump(out, fo, indent=1)
                        print(f"wrote {a.json}")
    return 0


if __name__ == "__main__":
    sys.exit(_main())
