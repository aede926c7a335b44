"""Selector calibration: measured candidates to a calibration file.

    python -m wide_reduction_reuse_amd.calibrate --out FILE [--sweep SWEEP.jsonl ...] [--run] [--base FILE]

With --run it first times every legal plan on the calibration shapes
(workloads.calibration_points(): the crossover sweep's operators, dtypes and
widths at 8, 64, 512 and 2048 MiB, sizes the scored sweep does not use; and
workloads.calibration_points_next(): the three further workloads at row counts
their width grid does not use; workloads.calibration_points_odd(): widths
2^k + 1, whose rows are not whole 16-byte vectors and run on tiles of their
own) with the sweep driver and writes the records to
the (one) --sweep file.  Several --sweep files are merged.  --ctrl FILE (the
output of ctrlbench.py; with --run it is measured first) adds the analytic
model's launch and per-row-wave exchange costs, fitted to the work-free
control kernel.  It then builds the table
credit_load_calibration reads: for each (op, dtype, cols) and each candidate
plan, the median kernel time at every calibrated row count.  The selector
interpolates these in (log rows, log time) for the rows it is asked about
(the CREDIT paper prices a schedule at the rate measured for it rather than a
device peak, Sec. III-D, Eq. 7; here every candidate is measured the same way).
The analytic model's streaming bandwidth is set to the best rate measured on
the largest calibration shapes.  --base FILE extends an existing calibration
file instead: its table rows are kept, the sweep records add rows, and a row
both hold gets, at each row count, the geometric mean of the two times (the
base's scalars, control-kernel costs and streaming rate are kept).  Base rows
of a plan the library no longer offers for their width (one it does not
enumerate, e.g. measured with an access width the planner no longer uses
there) are dropped.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
from collections import defaultdict

from .credit import DTYPES as DTS, OPS


# Table rows (version 3): [op, dt, cols, path, split_p, block, items, lds,
# vec_bytes, wgs_per_cu, n, rows_1, us_1, ...]; version 2 rows had no `lds`
# (register tiles only).
NKEY = 10


def upgrade_rows(doc: dict) -> list:
    """The table of a calibration document as version 3 rows."""
    if doc.get("version", 2) >= 3:
        return doc.get("table", [])
    return [r[:7] + [0] + r[7:] for r in doc.get("table", [])]


def upgrade_occupancy(doc: dict) -> list:
    """The occupancy rows of a calibration document in the version 3 layout
    [op, dt, kind, block, items, vec_bytes, row kind, lds, workgroups per CU]."""
    if doc.get("version", 2) >= 3:
        return doc.get("occupancy", [])
    return [r[:7] + [0] + r[7:] for r in doc.get("occupancy", [])]


def build_table(records):
    """One row per (op, dtype, cols, plan): the kernel time at every calibrated
    row count.  A shape timed in several sweeps (runs on different boxes)
    gets the geometric mean of its medians."""
    pts = defaultdict(lambda: defaultdict(list))
    for r in records:
        for c in r["candidates"]:
            p = c["plan"]
            key = (OPS[r["op"]], DTS[r["dtype"]], r["cols"], p["path"], p["split_p"], p["block_threads"],
                   p["items"], p.get("lds_items", 0), p["vec_bytes"], p["wgs_per_cu"])
            pts[key][r["rows"]].append(c["median_ms"] * 1000.0)
    table = []
    for key in sorted(pts):
        rows = sorted(pts[key])
        row = list(key) + [len(rows)]
        for n in rows:
            ts = pts[key][n]
            row += [n, round(math.exp(sum(math.log(t) for t in ts) / len(ts)), 4)]
        table.append(row)
    return table


def merge_tables(base, new):
    """Rows of `base` and `new` (build_table's format) keyed by their first
    NKEY fields; a key in both gets, per row count, the geometric mean of the
    two times, and the row counts only one of them measured as they are."""
    def points(row):
        n = row[NKEY]
        return {row[NKEY + 1 + 2 * i]: row[NKEY + 2 + 2 * i] for i in range(n)}
    merged = {tuple(r[:NKEY]): points(r) for r in base}
    for r in new:
        key = tuple(r[:NKEY])
        pts = points(r)
        if key in merged:
            old = merged[key]
            for n, t in pts.items():
                old[n] = round(math.sqrt(old[n] * t), 4) if n in old else t
        else:
            merged[key] = pts
    table = []
    for key in sorted(merged):
        pts = merged[key]
        row = list(key) + [len(pts)]
        for n in sorted(pts):
            row += [n, pts[n]]
        table.append(row)
    return table


def offered(row) -> bool:
    """Whether the library still enumerates the plan of a table row for its
    (op, dtype, cols), at the row's smallest calibrated row count."""
    from . import credit as C
    op, dt, cols, path, p, block, items, lds, vb, wpc = row[:NKEY]
    key = (op, dt, cols, row[NKEY + 1])
    if key not in _OFFERED:
        _OFFERED[key] = {(q.path, q.split_p, q.block_threads, q.items, q.lds_items, q.vec_bytes)
                         for q in C.credit_enumerate_plans(op, dt, row[NKEY + 1], cols)}
    return (path, p, block, items, lds, vb) in _OFFERED[key]


_OFFERED = {}


def unique_shapes(records) -> int:
    return len({(r["op"], r["dtype"], r["rows"], r["cols"]) for r in records})


def device_info():
    try:
        import torch
        if torch.cuda.is_available():
            p = torch.cuda.get_device_properties(0)
            return {"name": getattr(p, "gcnArchName", p.name), "cus": p.multi_processor_count}
    except Exception:
        pass
    return {}


def write_calibration(path: str, cal: dict) -> None:
    """The calibration file: scalars first, then one table row per line."""
    with open(path, "w") as f:
        f.write("{\n")
        f.write(' "version": 3,\n "source": %s,\n "stream_gbs": %s,\n' % (json.dumps(cal["source"]), cal["stream_gbs"]))
        for k in ("launch_us", "exchange_us"):
            if k in cal:
                f.write(' "%s": %s,\n' % (k, cal[k]))
        if "device" in cal:
            f.write(' "device": %s,\n' % json.dumps(cal["device"]))
        if "model" in cal:
            f.write(' "model": %s,\n' % json.dumps(cal["model"]))
        if "occupancy" in cal:
            f.write(' "occupancy": [\n')
            f.write(",\n".join("  " + json.dumps(row) for row in cal["occupancy"]))
            f.write("\n ],\n")
        f.write(' "table": [\n')
        f.write(",\n".join("  " + json.dumps(row) for row in cal["table"]))
        f.write("\n ]\n}\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--sweep", nargs="*", default=None, help="calibration sweep records (JSON lines)")
    ap.add_argument("--run", action="store_true", help="time the calibration shapes first (needs a GPU)")
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--ctrl", default=None, help="control-kernel fit (ctrlbench.py output)")
    ap.add_argument("--base", default=None, help="calibration file to extend with the sweep records")
    a = ap.parse_args(argv)
    if a.run:
        from . import sweep
        if not a.sweep or len(a.sweep) != 1:
            ap.error("--run needs one --sweep FILE for the records")
        rc = sweep.main(["--points", "calib_all", "--out", a.sweep[0], "--steps", str(a.steps)])
        if rc:
            return rc
        if a.ctrl:
            from . import ctrlbench
            rc = ctrlbench.main(["--out", a.ctrl, "--steps", str(a.steps)])
            if rc:
                return rc
    if not a.sweep:
        ap.error("--sweep FILE is required")
    records = [json.loads(l) for path in a.sweep for l in open(path) if l.strip()]
    if a.base:
        with open(a.base) as f:
            base = json.load(f)
        n_shapes = unique_shapes(records)
        cal = dict(base)
        base_rows = upgrade_rows(base)
        cal["occupancy"] = upgrade_occupancy(base)
        kept = [r for r in base_rows if offered(r)]
        if len(kept) != len(base_rows):
            print("dropped %d base rows of plans no longer offered" % (len(base["table"]) - len(kept)),
                  file=sys.stderr)
        cal["table"] = merge_tables(kept, build_table(records))
        cal["source"] = "%s; extended with %d more calibration shapes" % (base["source"], n_shapes)
        write_calibration(a.out, cal)
        print("wrote %s: %d candidates (%d from %s, %d shapes added)" % (a.out, len(cal["table"]), len(base["table"]),
                                                                        a.base, n_shapes), file=sys.stderr)
        return 0
    biggest = max(r["bytes"] for r in records)
    stream = max(r["bytes"] / (c["median_ms"] * 1e-3) / 1e9 for r in records if r["bytes"] == biggest
                 for c in r["candidates"])
    dev = device_info()
    n_shapes = unique_shapes(records)
    src = "median kernel times of every legal plan on %d calibration shapes" % n_shapes
    if len(records) > n_shapes:
        src += " (%d timed records, repeats averaged)" % len(records)
    cal = {"version": 3, "source": src,
           "stream_gbs": round(stream, 1), "table": build_table(records)}
    if a.ctrl:
        summ = [json.loads(l) for l in open(a.ctrl) if l.strip() and json.loads(l).get("summary")]
        if not summ:
            ap.error("%s has no summary line" % a.ctrl)
        cal["launch_us"] = summ[-1]["launch_us"]
        cal["exchange_us"] = summ[-1]["exchange_us"]
    if dev.get("cus"):
        cal["device"] = {"cus": dev["cus"]}
    write_calibration(a.out, cal)
    print("wrote %s: %d candidates over %d shapes (%d records)" % (a.out, len(cal["table"]), n_shapes, len(records)),
          file=sys.stderr)
    return 0


if __name__ == "__main__":
    sys.exit(main())
