"""Control-kernel timing for the selector's analytic terms.

    python -m wide_reduction_reuse_amd.ctrlbench [--out FILE] [--steps 15] [--warmup 3]

The CREDIT paper prices cluster overhead with a work-free control kernel: the
same grid, cluster size and synchronization as the clustered kernel but no
work, whose excess time over a one-wave control is T_ctrl (Sec. III-D, the
control-kernel term of Eq. 8).  Here the control twin of every split tile
(credit_control: tickets, exchange and reductions, no row loads or stores)
is timed at W = 1, 2, 4, 8 and 16 row waves per cluster (rows = C * W, C = the
clusters the device holds at once) and the medians are fitted by least
squares to T(W) = launch_us + W * exchange_us.  No data moves, so no cache
flush is needed between launches.

Writes one JSON line per (operator, P, tile) and a final summary line with
the medians over plans of the two constants; calibrate.py stores them as
launch_us and exchange_us of the analytic model.
"""
from __future__ import annotations

import argparse
import json
import sys

WAVES = (1, 2, 4, 8, 16)


def fit_line(xs, ys):
    """Least-squares (intercept, slope) of ys on xs."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx if sxx > 0 else 0.0
    return my - slope * mx, slope


def split_plans(C, op):
    """(P, plan, cols) for each compiled fp32 split tile of `op`: cols fill
    every slice of the tile exactly."""
    out = []
    for p_ in (2, 4, 8):
        for block, items in ((256, 8), (256, 16), (512, 4), (512, 8), (512, 16), (1024, 4), (1024, 8), (1024, 16)):
            plan = C.Plan.make(C.PATH_SPLIT_ROW, p_, block, items, 16, wgs_per_cu=0)
            cols = p_ * block * items * 4
            try:
                C.credit_occupancy(op, "f32", cols, plan)
            except C.CreditError:
                continue  # not compiled for this operator
            out.append((p_, plan, cols))
    return out


def time_control(C, HipEvents, op, rows, cols, plan, steps, warmup):
    import torch
    ev = HipEvents(warmup + steps)
    try:
        for i in range(warmup + steps):
            C.credit_control(op, rows, cols, "f32", plan, *ev.pairs[i])
        torch.cuda.synchronize()
        C.credit_check_errors()
        durs = sorted(ev.elapsed_ms(i) for i in range(warmup, warmup + steps))
    finally:
        ev.close()
    return durs[len(durs) // 2] * 1000.0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="-")
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--ops", nargs="*", default=["softmax", "layernorm", "rmsnorm", "softmax_bwd",
                                                  "layernorm_bwd", "quantize_int8"])
    a = ap.parse_args(argv)
    import torch
    from . import credit as C
    from .timing import HipEvents
    if not torch.cuda.is_available():
        print("ctrlbench needs a GPU", file=sys.stderr)
        return 2
    C.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = sys.stdout if a.out == "-" else open(a.out, "w")
    launches, exchanges = [], []
    for op in a.ops:
        for p_, plan, cols in split_plans(C, op):
            occ = C.credit_occupancy(op, "f32", cols, plan)
            clusters = max(1, occ * cus // p_)
            ts = [time_control(C, HipEvents, op, clusters * w, cols, plan, a.steps, a.warmup) for w in WAVES]
            launch, exch = fit_line(list(WAVES), ts)
            rec = {"op": op, "split_p": p_, "block_threads": plan.block_threads, "items": plan.items,
                   "clusters": clusters, "waves": list(WAVES), "us": [round(t, 3) for t in ts],
                   "launch_us": round(launch, 3), "exchange_us": round(exch, 3),
                   "t_ctrl_us_at_16": round(ts[-1] - ts[0], 3)}
            out.write(json.dumps(rec) + "\n")
            out.flush()
            launches.append(launch)
            exchanges.append(exch)
            print("[ctrl] %-14s P=%d %4dx%-2d C=%4d  T(W)=%s us  launch %.2f us, %.3f us per wave" %
                  (op, p_, plan.block_threads, plan.items, clusters, ["%.1f" % t for t in ts], launch, exch),
                  file=sys.stderr, flush=True)
    med = lambda v: sorted(v)[len(v) // 2]
    summary = {"summary": True, "plans": len(launches), "launch_us": round(med(launches), 3),
               "exchange_us": round(med(exchanges), 3)}
    out.write(json.dumps(summary) + "\n")
    if out is not sys.stdout:
        out.close()
    print("[ctrl] median launch %.3f us, exchange round %.3f us per row wave" %
          (summary["launch_us"], summary["exchange_us"]), file=sys.stderr)
    return 0


if __name__ == "__main__":
    sys.exit(main())
