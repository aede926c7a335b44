#!/usr/bin/env python3
"""Benchmark of the reduction-reuse hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all FILE]

A step is one call of the operator through the C ABI with the selector on
(CREDIT_PATH_AUTO: plan + the chosen kernel) over one batch of synthetic input
that is already resident in HBM.  Before every step an untimed 1 GiB
read-modify-write evicts L2 and the Infinity Cache, so the input is read from
HBM.  Each launch is bracketed by HIP events on the stream it runs on; the
flush queued ahead of it keeps host-side planning out of that interval.

Prints one JSON line: metric, value (algorithmic GB/s = one read of x + one
write of y + parameter vectors once, over the mean launch duration), the
roofline object for the kernel, and the CPU oracle's rate on the same workload.
With --all FILE it also writes one JSON line per (workload, path) to FILE.
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

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "layernorm_bf16_4096x8192"
FLUSH_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")


def csrc_hash() -> str:
    """Hash of the kernel sources: counter-derived traffic is only reported
    while the kernels it was measured on are unchanged."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "wide_reduction_reuse_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload)
    if not e or e.get("csrc_hash") != csrc_hash():
        return None
    return e


def upload(inp: W.HostInputs):
    import numpy as np
    import torch
    def dev(a):
        if a is None:
            return None
        if inp.workload.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()
    return dev(inp.x), dev(inp.gamma), dev(inp.beta)


def time_launches(fn, steps: int, warmup: int, flush_buf):
    """Run fn() warmup + steps times, each after an untimed cache flush;
    return (per-launch event durations in ms, wall seconds of the timed loop)."""
    import torch
    from wide_reduction_reuse_amd import credit as C
    for _ in range(warmup):
        C.credit_flush(flush_buf)
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        C.credit_flush(flush_buf)
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def run_workload(w: W.Workload, path: str, split_p: int, steps: int, warmup: int, flush_buf, inputs=None):
    import torch
    from wide_reduction_reuse_amd import credit as C
    inp = W.generate(w) if inputs is None else inputs
    x, g, b = upload(inp)
    y = torch.empty_like(x)

    def step():
        C.run(w.op, x, g, b, inp.eps, y=y, path=path, split_p=split_p)

    durs, wall = time_launches(step, steps, warmup, flush_buf)
    C.credit_check_errors()
    durs_sorted = sorted(durs)
    mean_ms = sum(durs) / len(durs)
    med_ms = durs_sorted[len(durs) // 2]
    return {"mean_ms": mean_ms, "median_ms": med_ms, "min_ms": durs_sorted[0], "wall_s": wall,
            "gbs": w.algorithmic_bytes() / (mean_ms * 1e-3) / 1e9,
            "gbs_median": w.algorithmic_bytes() / (med_ms * 1e-3) / 1e9}


def copy_ceiling(nbytes: int, steps: int, warmup: int, flush_buf):
    import torch
    from wide_reduction_reuse_amd import credit as C
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    durs, _ = time_launches(lambda: C.credit_copy(src, dst), steps, warmup, flush_buf)
    mean_ms = sum(durs) / len(durs)
    return {"bytes": 2 * nbytes, "mean_ms": mean_ms, "gbs": 2 * nbytes / (mean_ms * 1e-3) / 1e9}


def cpu_baseline(w: W.Workload, inp: W.HostInputs, repeats: int = 3):
    """The oracle, untuned, on the host cores: median of `repeats` runs."""
    import numpy as np
    import oracle
    def vals(a):
        if a is None:
            return None
        return oracle.bf16_bits_to_f64(a) if w.dtype == "bf16" else a.astype(np.float64)
    x, g, b = vals(inp.x), vals(inp.gamma), vals(inp.beta)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        if w.op == "softmax":
            oracle.softmax(x)
        elif w.op == "layernorm":
            oracle.layernorm(x, g, b, inp.eps)
        else:
            oracle.rmsnorm(x, g, inp.eps)
        times.append(time.perf_counter() - t0)
    t = sorted(times)[len(times) // 2]
    return {"value": round(w.algorithmic_bytes() / t / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "the full %dx%d workload, double precision, median of %d runs (%.2f s each)"
                      % (w.rows, w.cols, repeats, t)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.NAMED))
    ap.add_argument("--all", default=None, help="also time every workload and path; JSON lines to this file")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the row-wise operators shard by rows with no "
              "exchange between GPUs, so a multi-GPU figure would be N independent copies of "
              "this one; run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from wide_reduction_reuse_amd import credit as C
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    C.lib()
    flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda").zero_()

    w = W.NAMED[a.workload]
    inp = W.generate(w)
    plan = C.credit_select_path(w.op, w.dtype, w.rows, w.cols)
    r = run_workload(w, "auto", 0, a.steps, a.warmup, flush_buf, inputs=inp)
    achieved = w.algorithmic_bytes() / (r["mean_ms"] * 1e-3) / 1e9
    traffic = load_traffic(a.workload)
    result = {
        "metric": "achieved HBM GB/s (one read + one write) and % of MI355X peak per op/shape",
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
                   "median_ms": round(r["median_ms"], 5), "wall_s_timed_loop_incl_flush": round(r["wall_s"], 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"]},
    }
    if not a.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, inp)

    if a.all:
        with open(a.all, "w") as f:
            cc = copy_ceiling(128 << 20, a.steps, a.warmup, flush_buf)
            f.write(json.dumps({"kind": "copy_ceiling", **cc}) + "\n")
            f.flush()
            for name in W.CONFIG_ORDER:
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
