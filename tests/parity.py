"""Comparison of GPU outputs with the double-precision oracle, and the helpers
the GPU tests share (input upload, oracle evaluation with a per-session cache).

Tolerances (stated by the workload description, read as below):
  * fp32 outputs: e_i = |y_i - yhat_i| / max(|yhat_i|, tau) <= 1e-5 for every i,
    with tau = 2^-126 for softmax (purely relative: outputs are positive and
    well conditioned) and tau = 1 for LayerNorm and RMSNorm (outputs are unit
    scale; a relative bound is unattainable where yhat ~ 0 because any fp32 mean
    carries ~1 ulp of error that the cancellation in x - mean exposes).
  * bf16 outputs: r = the oracle rounded directly from double to bf16 (nearest,
    ties to even); pass iff every |y_i - r_i| <= 2e-2, or y_i and r_i are
    adjacent bf16 values (a one-ulp flip at a rounding midpoint, which an
    fp32-accurate result may land on the other side of when |y| >= 4, where one
    bf16 ulp exceeds 2e-2).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

import oracle
from wide_reduction_reuse_amd import workloads as W

FP32_TOL = 1e-5
BF16_ABS_TOL = 2e-2


@dataclasses.dataclass
class Verdict:
    ok: bool
    max_err: float          # the criterion's metric (fp32: e_i; bf16: |y - r| outside flips)
    max_abs: float          # literal max |y - yhat| (fp32) or |y - r| (bf16)
    max_rel: float          # literal max |y - yhat| / |yhat| (fp32 only)
    flips: int = 0          # bf16: one-ulp flips
    worst_index: int = -1

    def __str__(self):
        return ("ok=%s max_err=%.3g max_abs=%.3g max_rel=%.3g flips=%d worst=%d"
                % (self.ok, self.max_err, self.max_abs, self.max_rel, self.flips, self.worst_index))


def _bf16_ordered(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers whose order is the numeric order."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)


def compare(op: str, dtype: str, y_dev: np.ndarray, yhat: np.ndarray) -> Verdict:
    """y_dev: float32 array (f32) or uint16 bf16 bits (bf16), same shape as yhat (float64)."""
    yhat = np.asarray(yhat, dtype=np.float64)
    if dtype == "f32":
        y = np.asarray(y_dev, dtype=np.float32).astype(np.float64)
        tau = 2.0 ** -126 if op == "softmax" else 1.0
        diff = np.abs(y - yhat)
        e = diff / np.maximum(np.abs(yhat), tau)
        e = np.where(np.isnan(yhat) & np.isnan(y), 0.0, e)
        e = np.where(np.isnan(e), np.inf, e)
        worst = int(np.argmax(e)) if e.size else -1
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(yhat != 0, diff / np.abs(yhat), np.where(diff == 0, 0.0, np.inf))
        return Verdict(bool(e.size == 0 or e.max() <= FP32_TOL), float(e.max()) if e.size else 0.0,
                       float(np.nanmax(diff)) if diff.size else 0.0,
                       float(np.nanmax(rel)) if rel.size else 0.0, 0, worst)
    r_bits = oracle.round_bf16(yhat)
    y_bits = np.asarray(y_dev, dtype=np.uint16)
    r = oracle.bf16_bits_to_f64(r_bits)
    y = oracle.bf16_bits_to_f64(y_bits)
    diff = np.abs(y - r)
    diff = np.where(np.isnan(r) & np.isnan(y), 0.0, diff)
    diff = np.where(np.isnan(diff), np.inf, diff)
    adjacent = np.abs(_bf16_ordered(y_bits) - _bf16_ordered(r_bits)) <= 1
    bad = (diff > BF16_ABS_TOL) & ~adjacent
    flips = int(np.count_nonzero((diff > BF16_ABS_TOL) & adjacent))
    outside = np.where(adjacent & (diff > BF16_ABS_TOL), 0.0, diff)
    worst = int(np.argmax(outside)) if outside.size else -1
    return Verdict(not bool(bad.any()), float(outside.max()) if outside.size else 0.0,
                   float(diff.max()) if diff.size else 0.0, float("nan"), flips, worst)


# ---------------------------------------------------------------------------
# oracle evaluation on generated inputs (cached per workload for a session)
# ---------------------------------------------------------------------------
_ORACLE_CACHE: Dict[str, np.ndarray] = {}


def host_values(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    if a is None:
        return None
    return oracle.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def oracle_output(inp: W.HostInputs, cache: bool = True) -> np.ndarray:
    w = inp.workload
    key = "%s|%d|%d|%d" % (w.name, w.rows, w.cols, w.seed)
    if cache and key in _ORACLE_CACHE:
        return _ORACLE_CACHE[key]
    x = host_values(inp.x, w.dtype)
    if w.op == "softmax":
        yhat = oracle.softmax(x)
    elif w.op == "layernorm":
        yhat = oracle.layernorm(x, host_values(inp.gamma, w.dtype), host_values(inp.beta, w.dtype), inp.eps)
    else:
        yhat = oracle.rmsnorm(x, host_values(inp.gamma, w.dtype), inp.eps)
    if cache:
        _ORACLE_CACHE.clear()  # keep at most one large result alive
        _ORACLE_CACHE[key] = yhat
    return yhat


# ---------------------------------------------------------------------------
# device transfer (torch is used for device memory only)
# ---------------------------------------------------------------------------
def to_device(a: Optional[np.ndarray], dtype: str, device="cuda"):
    import torch
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
