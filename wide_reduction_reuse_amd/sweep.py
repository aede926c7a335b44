"""Exhaustive timing of every legal plan on a set of shapes.

    python -m wide_reduction_reuse_amd.sweep --points named|sweep|next|all|calib|calib_next|calib_next_more|calib_mid|calib_odd|calib_all|offgrid
                                             [--steps 15] [--warmup 3] [--ops ...] [--dtypes ...]
                                             [--min-cols N] [--odd-cols]

For each shape it enumerates the legal plans (credit_enumerate_plans: every
path 1 tile that holds the row, every path 3 tile, every (P, tile) of path 2),
times each one (median of `steps` flushed launches, dispatch timestamps) and
writes one JSON line per shape with all candidates, the selector's choice and
the model's predictions.  These records are the raw material of the selector
calibration and of its accuracy score (the CREDIT paper's evaluation times
every legal cluster size P and reports the fastest, Sec. IV-A; its
profitability accuracy compares predicted and measured winners, Sec. IV-C).

Inputs are synthetic and seeded: for timing, x (and dy, gamma, beta) are drawn
on the device with torch's seeded generator from the workload's distributions,
so that GiB-sized shapes need no host-side generation.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

from . import workloads as W
from .timing import flush_buffer, summarize, time_launches


def device_inputs(w: W.Workload) -> dict:
    """The operand mapping of w, inputs drawn on the device (W.device_inputs)."""
    return W.device_inputs(w)


def plan_key(p) -> str:
    key = "p%d-P%d-%dx%d-v%d-w%d" % (p.path, p.split_p, p.block_threads, p.items, p.vec_bytes, p.wgs_per_cu)
    return key + ("-l%d" % p.lds_items if p.lds_items else "")


def sweep_shape(w: W.Workload, steps: int, warmup: int, flush_buf) -> dict:
    import torch
    from . import credit as C
    t = device_inputs(w)
    sel = C.credit_select_path(w.op, w.dtype, w.rows, w.cols)
    cands = C.credit_enumerate_plans(w.op, w.dtype, w.rows, w.cols)
    rec = {"workload": w.name, "op": w.op, "dtype": w.dtype, "rows": w.rows, "cols": w.cols,
           "bytes": w.algorithmic_bytes(), "selected": plan_key(sel), "selected_plan": sel.as_dict(),
           "candidates": []}
    for p in cands:
        def launch(e0, e1, p=p):
            C.credit_run_plan_timed(w.op, p, t, e0, e1, eps=w.eps)
        durs, _ = time_launches(launch, steps, warmup, flush_buf)
        C.credit_check_errors()
        s = summarize(durs, w.algorithmic_bytes())
        rec["candidates"].append({"key": plan_key(p), "plan": p.as_dict(),
                                  "occupancy": C.credit_occupancy(w.op, w.dtype, w.cols, p),
                                  "predicted_us": p.predicted_us[p.path - 1], **s})
    best = min(rec["candidates"], key=lambda c: c["median_ms"])
    rec["best"] = best["key"]
    rec["best_median_ms"] = best["median_ms"]
    del t
    torch.cuda.empty_cache()
    return rec


def points(which: str, ops=None, min_cols: int = 0, dtypes=None, odd_cols=False):
    pts = []
    if which in ("named", "all"):
        pts += [W.NAMED[n] for n in W.CONFIG_ORDER + W.NEXT_ORDER]
    if which in ("sweep", "all"):
        pts += W.sweep_points()
    if which in ("next", "all"):
        pts += W.next_points()
    if which in ("calib", "calib_all"):
        pts += W.calibration_points()
    if which in ("calib_next", "calib_all"):
        pts += W.calibration_points_next()
    if which in ("calib_next_more", "calib_all"):
        pts += W.calibration_points_next_more()
    if which in ("calib_mid", "calib_all"):
        pts += W.calibration_points_mid()
    if which in ("calib_odd", "calib_all"):
        pts += W.calibration_points_odd()
    if which in ("calib_part", "calib_all"):
        pts += W.calibration_points_part()
    if which == "offgrid":
        pts += W.offgrid_points() + W.offgrid_points_next()
    if which == "lds":
        pts += W.lds_points()
    if ops:
        pts = [p for p in pts if p.op in ops]
    if dtypes:
        pts = [p for p in pts if p.dtype in dtypes]
    if odd_cols:
        pts = [p for p in pts if p.cols % 2 == 1]
    return [p for p in pts if p.cols >= min_cols]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--points", default="named", choices=("named", "sweep", "next", "all", "calib", "calib_next", "calib_next_more",
                                                         "calib_mid", "calib_odd", "calib_part", "calib_all",
                                                         "offgrid", "lds"))
    ap.add_argument("--ops", nargs="*", default=None)
    ap.add_argument("--min-cols", type=int, default=0, help="only shapes at least this wide")
    ap.add_argument("--dtypes", nargs="*", default=None, help="only these dtypes (f32, bf16)")
    ap.add_argument("--odd-cols", action="store_true", help="only shapes of odd width")
    ap.add_argument("--out", default="-")
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--warmup", type=int, default=3)
    a = ap.parse_args(argv)
    import torch
    from . import credit as C
    if not torch.cuda.is_available():
        print("the sweep needs a GPU", file=sys.stderr)
        return 2
    C.lib()
    flush_buf = flush_buffer()
    out = sys.stdout if a.out == "-" else open(a.out, "w")
    t0 = time.time()
    for w in points(a.points, a.ops, a.min_cols, a.dtypes, a.odd_cols):
        rec = sweep_shape(w, a.steps, a.warmup, flush_buf)
        out.write(json.dumps(rec) + "\n")
        out.flush()
        sel = next(c for c in rec["candidates"] if c["key"] == rec["selected"]) \
            if any(c["key"] == rec["selected"] for c in rec["candidates"]) else None
        print("[sweep %6.1fs] %-40s best %-22s %.4f ms  selected %-22s %s" %
              (time.time() - t0, w.name, rec["best"], rec["best_median_ms"], rec["selected"],
               "%.4f ms" % sel["median_ms"] if sel else "?"), file=sys.stderr, flush=True)
    if out is not sys.stdout:
        out.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
