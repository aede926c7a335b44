#!/usr/bin/env python3
"""Benchmark of the reduction-reuse hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--all FILE] [--no-cpu] [--path P --split-p N] [--no-copy] [--lnbwd-params]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM: the selector picks a plan for the shape
(credit_select_path, host only) and the chosen kernel runs it through the C ABI
(credit_run_plan_timed).  Before every step an untimed 1 GiB read-modify-write
evicts L2 and the Infinity Cache, so the input is read from HBM.

Timing: the library launches with hipExtLaunchKernel and a pair of HIP events
per step, which take the begin and end timestamps of the kernel dispatch
itself on the stream it runs on (the same interval rocprofv3's kernel trace
reports), so the flush, host-side planning and launch latency are outside it.

Prints one JSON line: metric, value (algorithmic GB/s = one read of every row
input + one write of the output + each parameter vector once, over the mean
kernel duration), the roofline object for the kernel, the CPU oracle's rate
on the same workload, and (in config) the rate of the library's streaming copy
of the same number of bytes, timed the same way.  --workload picks any named workload, including the three
further workloads (softmax-logits backward, LayerNorm backward, int8
quantization).  With --all FILE it also writes one JSON line per (workload,
path) and the streaming-copy ceiling to FILE.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from wide_reduction_reuse_amd import workloads as W  # noqa: E402
from wide_reduction_reuse_amd.timing import FLUSH_BYTES, summarize, time_launches  # noqa: E402

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "softmax_f32_256x262144"
PROFILES = os.path.join(ROOT, "profiles")
CPU_BASELINE_SECONDS = 10.0
METRIC = "achieved HBM GB/s (one read + one write) and % of MI355X peak per op/shape"


def csrc_hash() -> str:
    """Hash of the device-code sources (kernels, their headers and
    instantiations; not the host library): counter-derived traffic is only
    reported while the kernels it was measured on are unchanged."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "wide_reduction_reuse_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp")) and name != "planner.hpp":
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def plan_tag(plan) -> str:
    tag = "p%d-P%d-%dx%d" % (plan.path, plan.split_p, plan.block_threads, plan.items)
    return tag + ("+%d" % plan.lds_items if plan.lds_items else "")


def load_traffic(workload: str, plan):
    """The counter-derived HBM bytes per launch, if they were measured on the
    current kernels with the plan the selector now picks."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload)
    if not e or e.get("csrc_hash") != csrc_hash() or e.get("plan") != plan_tag(plan):
        return None
    return e


def run_workload(w: W.Workload, path: str, split_p: int, steps: int, warmup: int, flush_buf, inputs=None,
                 plan=None):
    """Time one workload.  path 'auto' runs the selector every step; a forced
    path (or an explicit plan) is planned once, as a caller forcing it would."""
    from wide_reduction_reuse_amd import credit as C
    inp = W.generate(w) if inputs is None else inputs
    t = W.alloc_outputs(w, W.to_device(inp))
    if plan is None and path != "auto":
        plan = C.credit_plan(w.op, w.dtype, w.rows, w.cols, path, split_p)

    def launch(e0, e1):
        p = plan if plan is not None else C.credit_select_path(w.op, w.dtype, w.rows, w.cols)
        C.credit_run_plan_timed(w.op, p, t, e0, e1, eps=inp.eps)

    durs, wall = time_launches(launch, steps, warmup, flush_buf)
    C.credit_check_errors()
    r = summarize(durs, w.algorithmic_bytes())
    r["wall_s"] = wall
    return r


def lnbwd_params(w: W.Workload, steps: int, warmup: int, flush_buf) -> dict:
    """Time LayerNorm backward's parameter part (both of its kernels) on the
    LayerNorm-backward workload w: algorithmic bytes = x and dy read once,
    the row statistics read, dgamma and dbeta written."""
    import torch
    from wide_reduction_reuse_amd import credit as C
    inp = W.generate(w)
    t = W.to_device(inp)
    _, stats = C.credit_layernorm_backward_stats(t["x"], t["dy"], t["gamma"], inp.eps)
    dg = torch.empty(w.cols, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)
    ws = torch.empty(max(16, C.credit_layernorm_backward_params_workspace(w.rows, w.cols, w.dtype)),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    durs, wall = time_launches(lambda e0, e1: C.credit_layernorm_backward_params(t["x"], t["dy"], stats, dg, db, ws),
                               steps, warmup, flush_buf, record_on=stream)
    eb = W.ELEM_BYTES[w.dtype]
    nbytes = w.rows * w.cols * 2 * eb + w.rows * 8 + 2 * w.cols * 4
    r = summarize(durs, nbytes)
    r["bytes"] = nbytes
    r["wall_s"] = wall
    return r


def copy_ceiling(nbytes: int, steps: int, warmup: int, flush_buf):
    import torch
    from wide_reduction_reuse_amd import credit as C
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    durs, _ = time_launches(lambda e0, e1: C.credit_copy(src, dst, e0, e1), steps, warmup, flush_buf)
    r = summarize(durs, 2 * nbytes)
    r["bytes"] = 2 * nbytes
    return r


def cpu_baseline(w: W.Workload, inp: W.HostInputs, seconds: float = CPU_BASELINE_SECONDS):
    """The oracle, untuned, on the host cores: repeated on the workload for
    about `seconds` of CPU time (at least 3 runs; a run is the whole workload
    when it takes under `seconds`, else the leading rows that fit), median."""
    import numpy as np
    import oracle

    def vals(a):
        if a is None:
            return None
        if w.op == "quantize_int8":  # the quantizer's oracle works in float32
            return oracle.bf16_bits_to_f32(a) if w.dtype == "bf16" else a
        return oracle.bf16_bits_to_f64(a) if w.dtype == "bf16" else a.astype(np.float64)

    def run(xs, dys):
        if w.op == "softmax":
            oracle.softmax(xs)
        elif w.op == "layernorm":
            oracle.layernorm(xs, g, b, inp.eps)
        elif w.op == "rmsnorm":
            oracle.rmsnorm(xs, g, inp.eps)
        elif w.op == "softmax_bwd":
            oracle.softmax_backward(xs, dys)
        elif w.op == "layernorm_bwd":
            oracle.layernorm_backward(xs, dys, g, inp.eps)
        else:
            oracle.quantize_int8(xs)

    g, b = vals(inp.gamma), vals(inp.beta)

    def sample(rows):
        return vals(inp.x[:rows]), (None if inp.dy is None else vals(inp.dy[:rows]))

    rows = min(w.rows, 64)
    xs, dys = sample(rows)
    t0 = time.perf_counter()
    run(xs, dys)
    t1 = time.perf_counter() - t0
    # bound the sample: the leading rows that take ~seconds/3 per run
    rows = max(1, min(w.rows, int(rows * (seconds / 3) / max(t1, 1e-9))))
    xs, dys = sample(rows)
    times = []
    start = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - start < seconds:
        t0 = time.perf_counter()
        run(xs, dys)
        times.append(time.perf_counter() - t0)
    t = sorted(times)[len(times) // 2]
    nbytes = w.with_shape(rows, w.cols).algorithmic_bytes()
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d of %d rows x %d cols, %s oracle (OpenMP over rows), median of %d runs "
                      "of %.4f s each over %.1f s" % (rows, w.rows, w.cols,
                                                       "float32" if w.op == "quantize_int8" else "float64",
                                                       len(times), t, time.perf_counter() - start)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.NAMED))
    ap.add_argument("--all", default=None, help="also time every named workload and path; JSON lines to FILE")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy", type=int, default=0, metavar="MIB",
                    help="only time the streaming-copy kernel on MIB MiB (the reference for counter scaling)")
    ap.add_argument("--path", default="auto", choices=("auto", "single", "split", "reread"),
                    help="force a path (for profiling one path; the default line uses the selector's plan)")
    ap.add_argument("--split-p", type=int, default=0, help="with --path split: workgroups per row (0 = chosen)")
    ap.add_argument("--no-copy", action="store_true", help="skip timing the streaming copy of the same bytes")
    ap.add_argument("--lnbwd-params", action="store_true",
                    help="only time LayerNorm backward's parameter part on the workload (a layernorm_bwd one)")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the row-wise operators shard by rows with no "
              "exchange between GPUs, and this build runs on a single MI355X; use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from wide_reduction_reuse_amd import credit as C
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    C.lib()
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda").zero_()
    if a.copy:
        cc = copy_ceiling(a.copy << 20, a.steps, a.warmup, flush_buf)
        print(json.dumps({"kind": "copy_ceiling", "mib": a.copy, **cc}), flush=True)
        return 0
    if a.lnbwd_params:
        w = W.NAMED[a.workload if W.NAMED[a.workload].op == "layernorm_bwd" else "layernorm_bwd_f32_2048x65536"]
        r = lnbwd_params(w, a.steps, a.warmup, flush_buf)
        print(json.dumps({"kind": "layernorm_bwd_params", "workload": w.name, "gbs": round(r["gbs"], 2),
                          "frac_of_peak": round(r["gbs"] / HBM_PEAK_GBS, 4), "bytes": r["bytes"],
                          "mean_ms": round(r["mean_ms"], 5), "median_ms": round(r["median_ms"], 5),
                          "timing": "HIP events recorded around both kernels on their stream"}), flush=True)
        return 0

    w = W.NAMED[a.workload]
    inp = W.generate(w)
    if a.path == "auto":
        plan = C.credit_select_path(w.op, w.dtype, w.rows, w.cols)
        r = run_workload(w, "auto", 0, a.steps, a.warmup, flush_buf, inputs=inp)
    else:
        plan = C.credit_plan(w.op, w.dtype, w.rows, w.cols, a.path, a.split_p)
        r = run_workload(w, a.path, a.split_p, a.steps, a.warmup, flush_buf, inputs=inp, plan=plan)
    achieved = r["gbs"]
    traffic = load_traffic(a.workload, plan)
    # the streaming copy of the same number of bytes (half read, half written),
    # timed the same way: the ceiling a kernel of this size can reach here
    copy = None if a.no_copy else copy_ceiling(w.algorithmic_bytes() // 2 // 16 * 16, a.steps, a.warmup, flush_buf)
    result = {
        "metric": METRIC,
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["mean_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "rows": w.rows, "cols": w.cols,
                   "path": plan.path, "split_p": plan.split_p, "block_threads": plan.block_threads,
                   "items": plan.items, "accumulate": "f32", "algorithmic_bytes": w.algorithmic_bytes(),
                   "cache_flush_bytes_between_steps": FLUSH_BYTES,
                   "median_ms": round(r["median_ms"], 5), "min_ms": round(r["min_ms"], 5),
                   "wall_s_timed_loop_incl_flush": round(r["wall_s"], 4),
                   "timing": "hipExtLaunchKernel dispatch timestamps",
                   "plan_forced": a.path != "auto",
                   "copy_same_bytes_gbs": None if copy is None else round(copy["gbs"], 2),
                   "frac_of_copy_same_bytes": None if copy is None else round(achieved / copy["gbs"], 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"]},
    }
    if not a.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, inp)

    if a.all:
        with open(a.all, "w") as f:
            for mib in (128, 256, 1024):
                cc = copy_ceiling(mib << 20, a.steps, a.warmup, flush_buf)
                f.write(json.dumps({"kind": "copy_ceiling", **cc}) + "\n")
                f.flush()
                print("[all] copy %d MiB %.1f GB/s (%.4f ms)" % (mib, cc["gbs"], cc["mean_ms"]),
                      file=sys.stderr, flush=True)
            for name in W.CONFIG_ORDER + W.NEXT_ORDER + W.EXTRA_ORDER:
                wk = W.NAMED[name]
                inpk = W.generate(wk)
                pl = C.credit_select_path(wk.op, wk.dtype, wk.rows, wk.cols)
                for path, p in [("auto", 0), ("single", 0), ("split", 2), ("split", 4), ("split", 8),
                                ("reread", 0)]:
                    try:
                        rk = run_workload(wk, path, p, a.steps, a.warmup, flush_buf, inputs=inpk)
                    except C.CreditError as e:
                        f.write(json.dumps({"workload": name, "path": path, "p": p, "error": str(e)}) + "\n")
                        continue
                    rec = {"workload": name, "path": path, "p": p, "selected": pl.as_dict(),
                           "frac_of_peak": round(rk["gbs"] / HBM_PEAK_GBS, 4), **rk}
                    f.write(json.dumps(rec) + "\n")
                    f.flush()
                    print("[all] %s %s P=%d %.1f GB/s (%.4f ms)" % (name, path, p, rk["gbs"], rk["mean_ms"]),
                          file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
