"""Fit the constants of the selector's analytic cost model to measured plans.

    python -m wide_reduction_reuse_amd.model_fit SWEEP.jsonl [...] [--from-table CALIB.json]
        [--base CALIB.json] [--out CALIB.json]

The model is the library's own (credit_enumerate_plans evaluated under a
calibration document that holds only the constants and the occupancy table),
so there is one implementation of it, in C++; this script only searches its
constants.  Inputs are sweep records (sweep.py: every legal plan of a shape
timed, each with the occupancy the HIP runtime reported for its kernel) and,
with --from-table, the measured points of a calibration table turned into
records of the same form.

Two stages, as the model has two parts (CREDIT paper, Sec. III-D):
  1. the streaming constants (achieved rate, bytes-in-flight latency, the
     reread's HBM share and efficiency, per-owner floor, launch cost,
     persistent-owner factor) by least squares on log(predicted / measured)
     over every path-1 and path-3 plan;
  2. the split control costs of Eq. 8 (one exchange per row wave, the split
     launch's fixed part) over the split plans the planner picks for each P
     (the model prices a P by the tile it would run), with stage 1's
     constants fixed.  The exchange-word rate of T_DSM is not fitted: at a few words
     per workgroup and row it is below the timings' noise, so it keeps its
     default.

--out writes --base (or an empty calibration) with its "model" and
"occupancy" sections replaced; its measured table is kept.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))

STREAM = ["bw_gbs", "lat_us", "owner_gbs", "miss3", "l0_us", "item_us", "own3_us", "launch_us", "eta3", "persist"]
SPLIT = ["exch_us", "split_launch_us"]
DEFAULTS = {"bw_gbs": 5100.5492, "lat_us": 0.6889, "owner_gbs": 44.5709, "miss3": 0.398, "l0_us": 2.2005,
            "item_us": 0.2123, "own3_us": 1.6787, "launch_us": 3.5074, "exch_us": 3.598,
            "split_launch_us": 6.2248, "eta3": 1.2562, "persist": 1.0084, "word_gbs": 10.0}
OPS = ["softmax", "layernorm", "rmsnorm", "softmax_bwd", "layernorm_bwd", "quantize_int8"]
DTS = ["f32", "bf16"]
KIND_WAVE, KIND_WG, KIND_SPLIT, KIND_REREAD = 1, 2, 3, 4


def plan_key(p: dict) -> tuple:
    return (p["path"], p["split_p"], p["block_threads"], p["items"], p.get("lds_items", 0), p["vec_bytes"],
            p["wgs_per_cu"])


def records_from_table(doc: dict) -> list:
    """One record per (op, dtype, cols, rows) that a calibration table measured,
    holding every candidate measured there (no occupancy: the table keeps none)."""
    from wide_reduction_reuse_amd.calibrate import NKEY, upgrade_rows
    shapes = {}
    for e in upgrade_rows(doc):
        op, dt, cols, path, p, block, items, lds, vb, wpc, n = e[:NKEY + 1]
        plan = {"path": path, "split_p": p, "block_threads": block, "items": items, "lds_items": lds,
                "vec_bytes": vb, "wgs_per_cu": wpc}
        for j in range(n):
            rows, us = e[NKEY + 1 + 2 * j], e[NKEY + 2 + 2 * j]
            shapes.setdefault((op, dt, cols, int(rows)), []).append({"plan": plan, "median_ms": us / 1e3})
    return [{"workload": "table_%s_%s_%dx%d" % (OPS[op], DTS[dt], rows, cols), "op": OPS[op], "dtype": DTS[dt],
             "rows": rows, "cols": cols, "candidates": c} for (op, dt, cols, rows), c in shapes.items()]


def row_kind(op: str, dt: str, cols: int, path: int = 1) -> int:
    """The held register tiles' row kind for this width on `path` (1 or 2;
    the library's held_row_kind): 2 for rows whose byte length is not a
    multiple of 64 (held from the 64-byte line below their start) of softmax,
    softmax backward, the quantizer and RMSNorm, of fp32 LayerNorm backward on
    path 1 when the byte length is a multiple of 16, and of LayerNorm when the
    byte length is not a multiple of 4; 1 for the other rows of LayerNorm and
    fp32 LayerNorm backward whose byte length is a multiple of 4 but not of 16
    (a partial last vector); else 0.  bf16 LayerNorm backward: 2 on path 1
    for rows that are not whole 16-byte vectors, else 0."""
    nbytes = cols * (4 if dt == "f32" else 2)
    if op == "layernorm_bwd":
        if dt != "f32":
            return 2 if path == 1 and nbytes % 16 else 0
        if nbytes % 16:
            return 1
        return 2 if path == 1 and nbytes % 64 else 0
    if op == "layernorm":
        if nbytes % 4:
            return 2
        return 1 if nbytes % 16 else 0
    return 2 if nbytes % 64 else 0


def occupancy_table(C, records) -> list:
    """[op, dt, kind, block, items, vec_bytes, row kind, lds, workgroups per
    CU] for every kernel whose occupancy the records hold."""
    table = {}
    for r in records:
        for c in r["candidates"]:
            occ = c.get("occupancy")
            if not occ:
                continue
            p = c["plan"]
            path = p["path"]
            kind = {2: KIND_SPLIT, 3: KIND_REREAD}.get(path, KIND_WAVE if p["block_threads"] == 64 else KIND_WG)
            part = 0 if path == 3 or p.get("lds_items", 0) else row_kind(r["op"], r["dtype"], r["cols"], path)
            key = (OPS.index(r["op"]), DTS.index(r["dtype"]), kind, p["block_threads"], p["items"],
                   p["vec_bytes"], part, p.get("lds_items", 0))
            table[key] = int(occ)
    return [list(k) + [v] for k, v in sorted(table.items())]


class Evaluator:
    """Predicted times of the records' candidates under a set of constants,
    from the library (one load of a model-only calibration per evaluation)."""

    def __init__(self, C, records, occupancy, device=None):
        self.C = C
        self.records = records
        self.occupancy = occupancy
        self.device = device

    def load(self, consts: dict, peak: bool = False) -> None:
        doc = {"version": 3, "model": consts, "occupancy": self.occupancy}
        if self.device:
            doc["device"] = self.device
        if peak:
            doc["model_peak_bandwidth"] = 1
        with tempfile.NamedTemporaryFile("w", suffix=".json", delete=False) as f:
            json.dump(doc, f)
        try:
            self.C.credit_load_calibration(f.name)
        finally:
            os.unlink(f.name)

    def pairs(self, consts: dict, paths) -> list:
        """(predicted us, measured us) for every candidate on `paths` that the
        planner still enumerates."""
        self.load(consts)
        out = []
        for r in self.records:
            plans = [q.as_dict() for q in self.C.credit_enumerate_plans(r["op"], r["dtype"], r["rows"], r["cols"])]
            pred = {plan_key(p): p["predicted_us"][p["path"] - 1] for p in plans}
            for c in r["candidates"]:
                if c["plan"]["path"] not in paths:
                    continue
                us = pred.get(plan_key(c["plan"]))
                if us is not None and us > 0 and c["median_ms"] > 0:
                    out.append((us, c["median_ms"] * 1e3))
        return out

    def split_pairs(self, consts: dict) -> list:
        """(predicted us, measured us) of the split plan the planner picks for
        each P: the model prices each P by the tile it would run."""
        self.load(consts)
        out = []
        for r in self.records:
            meas = {plan_key(c["plan"]): c["median_ms"] * 1e3 for c in r["candidates"] if c["plan"]["path"] == 2}
            if not meas:
                continue
            for p in (2, 4, 8):
                try:
                    plan = self.C.credit_plan(r["op"], r["dtype"], r["rows"], r["cols"], "split", p).as_dict()
                except self.C.CreditError:
                    continue
                m = meas.get(plan_key(plan))
                if m and plan["predicted_us"][1] > 0:
                    out.append((plan["predicted_us"][1], m))
        return out


def fit(C, records, occupancy, start: dict | None = None, device=None, log=print) -> dict:
    import numpy as np
    from scipy.optimize import least_squares
    ev = Evaluator(C, records, occupancy, device)
    consts = dict(DEFAULTS)
    consts.update(start or {})

    def stage(names, paths):
        x0 = np.log([consts[k] for k in names])

        def resid(x):
            trial = dict(consts)
            trial.update(zip(names, np.exp(x)))
            got = ev.split_pairs(trial) if paths == (2,) else ev.pairs(trial, paths)
            return np.array([math.log(p / m) for p, m in got])
        r0 = resid(x0)
        if len(r0) <= len(names):
            log("stage %s: %d plans, too few to fit; constants kept" % ("/".join(map(str, paths)), len(r0)))
            return
        res = least_squares(resid, x0, method="trf", x_scale=1.0, diff_step=1e-3, max_nfev=60 * len(names))
        consts.update(zip(names, (float(v) for v in np.exp(res.x))))
        log("stage %s: %d plans, rms log error %.4f -> %.4f" % (
            "/".join(map(str, paths)), len(r0), math.sqrt(float(np.mean(r0 ** 2))),
            math.sqrt(float(np.mean(res.fun ** 2)))))
    stage(STREAM, (1, 3))
    stage(SPLIT, (2,))
    return {k: round(v, 6) for k, v in consts.items()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("sweep", nargs="*", help="sweep records (sweep.py) to fit to; their occupancy fields "
                    "make the occupancy table")
    ap.add_argument("--occupancy-from", nargs="*", default=[], help="further sweep records whose occupancy "
                    "fields join the table (not fitted to)")
    ap.add_argument("--from-table", default=None, help="also fit to the measured points of this calibration table")
    ap.add_argument("--base", default=None, help="calibration whose table and device the output keeps")
    ap.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    sys.path.insert(0, os.path.dirname(PKG))
    from wide_reduction_reuse_amd import credit as C
    records = [json.loads(l) for path in a.sweep for l in open(path) if l.strip()]
    records = [r for r in records if "candidates" in r]
    extra = [json.loads(l) for path in a.occupancy_from for l in open(path) if l.strip()]
    C.credit_load_calibration(None)
    occupancy = occupancy_table(C, records + [r for r in extra if "candidates" in r])
    if a.from_table:
        records += records_from_table(json.load(open(a.from_table)))
    base = json.load(open(a.base)) if a.base else {"version": 2}
    print("fitting to %d shapes; occupancy of %d kernels" % (len(records), len(occupancy)))
    consts = fit(C, records, occupancy, start=base.get("model"), device=base.get("device"))
    print(json.dumps(consts))
    if a.out:
        from wide_reduction_reuse_amd.calibrate import upgrade_rows, write_calibration
        base["table"] = upgrade_rows(base)
        base["version"] = 3
        base["model"] = consts
        base["occupancy"] = occupancy
        base.setdefault("source", "model constants only")
        base.setdefault("stream_gbs", consts["bw_gbs"])
        base.setdefault("table", [])
        write_calibration(a.out, base)
        print("wrote", a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
