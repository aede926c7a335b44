"""Summaries of rocprofv3 CSV output for the profiles kept with the sources.

    python -m wide_reduction_reuse_amd.rocprof_summary stats DIR
        per-kernel call count and average / min / max duration from a
        --kernel-trace --stats run (the *_kernel_stats.csv file in DIR)
    python -m wide_reduction_reuse_amd.rocprof_summary pmc DIR [KERNEL_SUBSTRING]
        per-kernel average of each counter over its dispatches from a --pmc run
        (the *_counter_collection.csv file in DIR)
    python -m wide_reduction_reuse_amd.rocprof_summary traffic OUT.json WORKLOAD KERNEL_SUBSTR \\
        FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR COPY_BYTES CSRC_HASH PLAN_TAG
        HBM bytes per launch of the kernel: FETCH_SIZE and WRITE_SIZE (KiB per
        dispatch) of the kernel, each scaled by bytes / counter of the streaming
        copy kernel on COPY_BYTES read + COPY_BYTES written; merged into OUT.json
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys
from collections import defaultdict


def _one(dirname: str, pattern: str) -> str:
    files = sorted(glob.glob(os.path.join(dirname, "**", pattern), recursive=True))
    if not files:
        raise SystemExit("no %s under %s" % (pattern, dirname))
    return files[0]


def stats(dirname: str):
    path = _one(dirname, "*kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        out.append({"kernel": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                    "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                    "percent": float(r["Percentage"])})
    return out


def pmc(dirname: str, kernel_sub: str = ""):
    path = _one(dirname, "*counter_collection.csv")
    acc = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(path)):
        name = r.get("Kernel_Name", "")
        if kernel_sub and kernel_sub not in name:
            continue
        acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: {"mean": sum(v) / len(v), "n": len(v), "min": min(v), "max": max(v)} for c, v in d.items()}
            for k, d in acc.items()}


def _counter(dirname: str, kernel_sub: str, counter: str) -> float:
    res = pmc(dirname, kernel_sub)
    vals = [d[counter]["mean"] for d in res.values() if counter in d]
    if not vals:
        raise SystemExit("no %s for %r under %s" % (counter, kernel_sub, dirname))
    if len(vals) > 1:
        raise SystemExit("%r matches %d kernels under %s" % (kernel_sub, len(vals), dirname))
    return vals[0]


def traffic(out_json, workload, kernel_sub, fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes, csrc_hash,
            plan_tag):
    copy_bytes = float(copy_bytes)
    cf = _counter(cfetch_dir, "copy_kernel", "FETCH_SIZE")
    cw = _counter(cwrite_dir, "copy_kernel", "WRITE_SIZE")
    f = _counter(fetch_dir, kernel_sub, "FETCH_SIZE")
    w = _counter(write_dir, kernel_sub, "WRITE_SIZE")
    sf, sw = copy_bytes / cf, copy_bytes / cw
    rec = {"kernel": kernel_sub, "csrc_hash": csrc_hash, "plan": plan_tag,
           "fetch_kib": f, "write_kib": w, "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": copy_bytes,
           "scale_fetch": sf, "scale_write": sw,
           "fetch_bytes": f * sf, "write_bytes": w * sw, "bytes_per_launch": f * sf + w * sw}
    data = json.load(open(out_json)) if os.path.exists(out_json) else {}
    data[workload] = rec
    with open(out_json, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    return rec


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if not argv:
        print(__doc__)
        return 2
    cmd = argv[0]
    if cmd == "stats":
        for r in stats(argv[1]):
            print("%-100s calls=%4d avg=%10.1f ns min=%10.1f max=%10.1f %5.1f%%" %
                  (r["kernel"][:100], r["calls"], r["avg_ns"], r["min_ns"], r["max_ns"], r["percent"]))
    elif cmd == "pmc":
        res = pmc(argv[1], argv[2] if len(argv) > 2 else "")
        for k, d in res.items():
            for c, v in d.items():
                print("%-100s %-24s mean=%14.1f n=%d min=%.1f max=%.1f" % (k[:100], c, v["mean"], v["n"],
                                                                          v["min"], v["max"]))
    elif cmd == "traffic":
        print(json.dumps(traffic(*argv[1:11]), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main())
