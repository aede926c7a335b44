"""Score the selector against exhaustive timing.

    python -m wide_reduction_reuse_amd.selector_eval SWEEP.jsonl [SWEEP2.jsonl ...]
        [--model calibrated|analytic|peak] [--calib FILE] [--prefix P] [--md OUT.md] [--crossover]

For each shape of a sweep (every legal plan timed, sweep.py), ask the
selector (credit_select_path, host only) for its plan and compare its
measured median with the fastest candidate's.  Reported, as the CREDIT paper
reports profitability accuracy against measurement (Sec. IV-C, Table V):

  * primary: the selected plan is within max(1%, 2 x its coefficient of
    variation) of the fastest measured plan;
  * strict: the selected plan is the fastest measured plan;
  * split vs non-split: the selector's prediction of whether the best split
    plan beats the best non-split plan matches the measurement (shapes where
    a split is legal).

Models (--model): `calibrated` (the calibration file's measured candidates,
analytic elsewhere), `analytic` (the cost model alone: the calibration's
fitted constants and kernel occupancy table, none of its measured
candidates), `peak` (the same with streaming priced at the device's peak HBM
bandwidth: the ablation of the paper's
Table V, first row; the paper's second ablated term, a shared-memory deposit
serialized behind the input load, has no counterpart here because held rows
are loaded straight into registers).

--crossover also reports, per (operator, dtype, input size) series of widths,
the smallest width at which splitting is measured to beat the best non-split
plan and the smallest at which the model predicts it (the crossover-width test
of the paper's Fig. 4).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
DEFAULT_CALIB = os.path.join(PKG, "calib", "mi355x.json")


def key_of(p: dict) -> tuple:
    return (p["path"], p["split_p"], p["block_threads"], p["items"], p["vec_bytes"], p["wgs_per_cu"],
            p.get("lds_items", 0))


def evaluate(records, C):
    rows = []
    for r in records:
        plan = C.credit_select_path(r["op"], r["dtype"], r["rows"], r["cols"]).as_dict()
        cands = r["candidates"]
        best = min(cands, key=lambda c: c["median_ms"])
        sel = next((c for c in cands if key_of(c["plan"]) == key_of(plan)), None)
        split = [c for c in cands if c["plan"]["path"] == 2]
        rec = {"workload": r["workload"], "best": best["median_ms"], "best_plan": key_of(best["plan"]),
               "selected_plan": key_of(plan), "selected": sel["median_ms"] if sel else None}
        rec["ratio"] = rec["selected"] / rec["best"] if sel else float("inf")
        tol = max(0.01, 2.0 * sel.get("cov", 0.0)) if sel else 0.0
        rec["ok"] = sel is not None and sel["median_ms"] <= best["median_ms"] * (1.0 + tol)
        rec["strict"] = sel is not None and sel["median_ms"] == best["median_ms"]
        if split:
            meas = min(c["median_ms"] for c in split) < min(c["median_ms"] for c in cands if c["plan"]["path"] != 2)
            pu = plan["predicted_us"]
            pred_split = pu[1]
            pred_other = min([v for v in (pu[0], pu[2]) if v >= 0] or [float("inf")])
            rec["split_meas"] = meas
            rec["split_pred"] = pred_split >= 0 and pred_split < pred_other
            rec["split_ok"] = rec["split_pred"] == meas
        rows.append(rec)
    return rows


def summary(rows) -> dict:
    n = len(rows)
    sp = [r for r in rows if "split_ok" in r]
    return {"shapes": n, "primary": sum(r["ok"] for r in rows), "strict": sum(r["strict"] for r in rows),
            "split_shapes": len(sp), "split_ok": sum(r["split_ok"] for r in sp),
            "geomean_selected_over_best": _geomean([r["ratio"] for r in rows])}


def crossover(records, rows_eval):
    """Per series (op, dtype, size class): widths ascending with measured and
    predicted split profitability; the crossover is the smallest width from
    which on the split stays profitable."""
    series = {}
    for r, e in zip(records, rows_eval):
        if "split_ok" not in e:
            continue
        size = r["rows"] * r["cols"]
        key = (r["op"], r["dtype"], size if "sweep" in r["workload"] else r["rows"])
        series.setdefault(key, []).append((r["cols"], e["split_meas"], e["split_pred"]))
    out = []
    for key in sorted(series):
        pts = sorted(series[key])

        def first_stable(flags):
            for i in range(len(pts)):
                if all(f for f in flags[i:]):
                    return pts[i][0]
            return None
        meas = first_stable([m for _, m, _ in pts])
        pred = first_stable([p for _, _, p in pts])
        widths = [c for c, _, _ in pts]
        if meas == pred:
            d = 0
        elif meas is None or pred is None:
            d = None
        else:
            d = widths.index(pred) - widths.index(meas)
        out.append({"series": "%s %s %s" % key, "widths": widths, "measured": meas, "predicted": pred,
                    "steps_off": d})
    return out


def _geomean(v):
    import math
    v = [x for x in v if x != float("inf")]
    return math.exp(sum(math.log(x) for x in v) / len(v)) if v else float("nan")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("sweep", nargs="+")
    ap.add_argument("--model", default="calibrated", choices=("calibrated", "analytic", "peak"))
    ap.add_argument("--calib", default=DEFAULT_CALIB, help="calibration file (its table is used by "
                    "--model calibrated, its measured copy rate by --model analytic)")
    ap.add_argument("--md", default=None)
    ap.add_argument("--prefix", default="sweep", help="score only workloads whose name starts with this")
    ap.add_argument("--crossover", action="store_true")
    a = ap.parse_args(argv)
    sys.path.insert(0, os.path.dirname(PKG))
    import tempfile
    from wide_reduction_reuse_amd import credit as C
    if a.model == "calibrated":
        C.credit_load_calibration(a.calib)
    else:
        base = json.load(open(a.calib))
        from wide_reduction_reuse_amd.calibrate import upgrade_occupancy
        model = {"version": 3, "occupancy": upgrade_occupancy(base)}
        for k in ("device", "model"):
            if k in base:
                model[k] = base[k]
        if a.model == "peak":
            model["model_peak_bandwidth"] = 1
        with tempfile.NamedTemporaryFile("w", suffix=".json", delete=False) as f:
            json.dump(model, f)
        C.credit_load_calibration(f.name)
        os.unlink(f.name)
    records = [json.loads(l) for path in a.sweep for l in open(path) if l.strip()]
    records = [r for r in records if r["workload"].startswith(a.prefix)]
    rows = evaluate(records, C)
    s = summary(rows)
    s["model"] = a.model
    print(json.dumps(s))
    if a.crossover:
        for c in crossover(records, rows):
            print(json.dumps(c))
    if a.md:
        with open(a.md, "w") as f:
            f.write("| shape | selected | ms | fastest | ms | ratio | ok |\n|---|---|---|---|---|---|---|\n")
            for r in rows:
                f.write("| %s | %s | %s | %s | %.4f | %.3f | %s |\n" % (
                    r["workload"], r["selected_plan"], "%.4f" % r["selected"] if r["selected"] else "-",
                    r["best_plan"], r["best"], r["ratio"], "yes" if r["ok"] else "NO"))
    return 0


if __name__ == "__main__":
    sys.exit(main())
