"""Kernel timing helpers shared by bench.py and the sweep driver.

Kernels are launched through the library with a pair of HIP events that take
the dispatch's own begin and end timestamps (hipExtLaunchKernel), so an
interval is device execution time only.  Before every timed launch an untimed
read-modify-write of a 1 GiB buffer evicts L2 and the Infinity Cache.
"""
from __future__ import annotations

import ctypes
import time

FLUSH_BYTES = 1 << 30


class HipEvents:
    """Pairs of timing-enabled hipEvent_t from the HIP runtime torch loaded."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a.value, b.value))

    def record(self, event: int, stream: int) -> None:
        """Record `event` on `stream` (for launches that take no events)."""
        if self.hip.hipEventRecord(event, stream):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int) -> float:
        a, b = self.pairs[i]
        if self.hip.hipEventSynchronize(b):
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b):
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        self.pairs = []


def flush_buffer():
    import torch
    return torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")


def time_launches(launch, steps: int, warmup: int, flush_buf, record_on=None):
    """Call launch(start_event, stop_event) warmup + steps times, each after an
    untimed cache flush; return the per-step kernel durations (ms) of the
    timed steps and the wall seconds of the timed loop.  With record_on (a
    stream handle), the events are recorded on that stream around
    launch(None, None) instead (work of several kernels, then the interval
    includes the gaps between them)."""
    import torch
    from . import credit as C
    ev = HipEvents(warmup + steps)
    if record_on is not None:
        inner = launch

        def launch(e0, e1):
            ev.record(e0, record_on)
            inner(None, None)
            ev.record(e1, record_on)
    try:
        for i in range(warmup):
            C.credit_flush(flush_buf)
            launch(*ev.pairs[i])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warmup, warmup + steps):
            C.credit_flush(flush_buf)
            launch(*ev.pairs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        durs = [ev.elapsed_ms(i) for i in range(warmup, warmup + steps)]
    finally:
        ev.close()
    return durs, wall


def summarize(durs, nbytes: int) -> dict:
    s = sorted(durs)
    mean_ms = sum(durs) / len(durs)
    med_ms = s[len(s) // 2]
    var = sum((d - mean_ms) ** 2 for d in durs) / max(1, len(durs) - 1)
    return {"mean_ms": mean_ms, "median_ms": med_ms, "min_ms": s[0], "max_ms": s[-1],
            "cov": (var ** 0.5) / mean_ms if mean_ms > 0 else 0.0,
            "gbs": nbytes / (mean_ms * 1e-3) / 1e9, "gbs_median": nbytes / (med_ms * 1e-3) / 1e9}
