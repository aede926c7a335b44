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
  * the two backward operators: each output is a small difference of larger
    terms (p_i (dy_i - dot); rstd (g_i - mean g - xhat_i mean(g xhat))), whose
    sums (dot, mean g, mean(g xhat)) may themselves cancel.  The rounding error
    of a sum is bounded in proportion to the sum of its terms' magnitudes, so
    the fp32 criterion takes tau_i = that magnitude instead of 1: softmax
    backward tau_i = phat_i (|dy_i| + sum_j |dy_j| phat_j); LayerNorm backward
    tau_i = rstd (|g_i| + mean |g| + |xhat_i| mean |g xhat|).  bf16 outputs of
    the backward operators (softmax backward's values are mostly far below
    2e-2, so that the absolute rule alone would check nothing) must in
    addition be within one bf16 ulp of r, or within 2^-8 |yhat_i| +
    1e-5 tau_i of yhat.
  * int8 quantization: codes and per-row scales bit-exact (both sides decide
    them in the same fp32 arithmetic).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import warnings

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


def compare(op: str, dtype: str, y_dev: np.ndarray, yhat: np.ndarray, tau_elem: Optional[np.ndarray] = None) -> Verdict:
    """y_dev: float32 array (f32) or uint16 bf16 bits (bf16), same shape as yhat
    (float64); tau_elem: per-element tolerance scale (backward operators)."""
    yhat = np.asarray(yhat, dtype=np.float64)
    if dtype == "f32":
        y = np.asarray(y_dev, dtype=np.float32).astype(np.float64)
        tau = tau_elem if tau_elem is not None else (2.0 ** -126 if op == "softmax" else 1.0)
        diff = np.abs(y - yhat)
        # an exact match is no error, also where the scale is zero (a
        # backward operator's tau where the probability underflows to 0)
        with np.errstate(divide="ignore", invalid="ignore"):
            e = np.where(diff == 0, 0.0, diff / np.maximum(np.abs(yhat), tau))
        e = np.where(np.isnan(yhat) & np.isnan(y), 0.0, e)
        e = np.where(np.isnan(e), np.inf, e)
        worst = int(np.argmax(e)) if e.size else -1
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(yhat != 0, diff / np.abs(yhat), np.where(diff == 0, 0.0, np.inf))
        with warnings.catch_warnings():  # all-NaN rows only make the reported maxima NaN
            warnings.simplefilter("ignore", RuntimeWarning)
            max_abs = float(np.nanmax(diff)) if diff.size else 0.0
            max_rel = float(np.nanmax(rel)) if rel.size else 0.0
        return Verdict(bool(e.size == 0 or e.max() <= FP32_TOL), float(e.max()) if e.size else 0.0,
                       max_abs, max_rel, 0, worst)
    r_bits = oracle.round_bf16(yhat)
    y_bits = np.asarray(y_dev, dtype=np.uint16)
    r = oracle.bf16_bits_to_f64(r_bits)
    y = oracle.bf16_bits_to_f64(y_bits)
    diff = np.abs(y - r)
    diff = np.where(np.isnan(r) & np.isnan(y), 0.0, diff)
    diff = np.where(np.isnan(diff), np.inf, diff)
    adjacent = np.abs(_bf16_ordered(y_bits) - _bf16_ordered(r_bits)) <= 1
    bad = (diff > BF16_ABS_TOL) & ~adjacent
    if tau_elem is not None:
        close = np.abs(y - yhat) <= 2.0 ** -8 * np.abs(yhat) + FP32_TOL * tau_elem
        bad |= ~adjacent & ~close
    flips = int(np.count_nonzero((diff > BF16_ABS_TOL) & adjacent))
    outside = np.where(adjacent & (diff > BF16_ABS_TOL), 0.0, diff)
    worst = int(np.argmax(outside)) if outside.size else -1
    return Verdict(not bool(bad.any()), float(outside.max()) if outside.size else 0.0,
                   float(diff.max()) if diff.size else 0.0, float("nan"), flips, worst)


# ---------------------------------------------------------------------------
# oracle evaluation on generated inputs (cached per workload for a session)
# ---------------------------------------------------------------------------
_ORACLE_CACHE: Dict[str, object] = {}


def host_values(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    if a is None:
        return None
    return oracle.bf16_bits_to_f64(a) if dtype == "bf16" else a.astype(np.float64)


def oracle_output(inp: W.HostInputs, cache: bool = True, rows=None):
    """The oracle's result on inp (or on the row indices `rows` of it): a float64
    array, or for quantization the pair (int8 codes, float32 scales)."""
    w = inp.workload
    key = "%s|%d|%d|%d|%s" % (w.name, w.rows, w.cols, w.seed, None if rows is None else hash(tuple(rows)))
    if cache and key in _ORACLE_CACHE:
        return _ORACLE_CACHE[key]
    sel = (lambda a: a) if rows is None else (lambda a: None if a is None else a[rows])
    g = host_values(inp.gamma, w.dtype)
    b = host_values(inp.beta, w.dtype)
    if w.op == "quantize_int8":
        xs = sel(inp.x)
        out = oracle.quantize_int8(oracle.bf16_bits_to_f32(xs) if w.dtype == "bf16" else xs)
    else:
        x = host_values(sel(inp.x), w.dtype)
        dy = host_values(sel(inp.dy), w.dtype)
        if w.op == "softmax":
            out = oracle.softmax(x)
        elif w.op == "layernorm":
            out = oracle.layernorm(x, g, b, inp.eps)
        elif w.op == "rmsnorm":
            out = oracle.rmsnorm(x, g, inp.eps)
        elif w.op == "softmax_bwd":
            out = oracle.softmax_backward(x, dy)
        elif w.op == "layernorm_bwd":
            out = oracle.layernorm_backward(x, dy, g, inp.eps)
        else:
            raise ValueError(w.op)
    if cache:
        _ORACLE_CACHE.clear()  # keep at most one large result alive
        _ORACLE_CACHE[key] = out
    return out


def tolerance_scale(inp: W.HostInputs, rows=None) -> Optional[np.ndarray]:
    """Per-element magnitude of the terms whose difference a backward output
    is (see the module docstring); None for the other operators."""
    w = inp.workload
    if w.op not in ("softmax_bwd", "layernorm_bwd"):
        return None
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    x = host_values(sel(inp.x), w.dtype)
    dy = host_values(sel(inp.dy), w.dtype)
    if w.op == "softmax_bwd":
        p = oracle.softmax(x)
        return p * (np.abs(dy) + (np.abs(dy) * p).sum(axis=1, keepdims=True))
    gam = host_values(inp.gamma, w.dtype)
    mu = x.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=1, keepdims=True) + inp.eps)
    xhat = (x - mu) * rstd
    g = gam * dy
    return rstd * (np.abs(g) + np.abs(g).mean(axis=1, keepdims=True) +
                   np.abs(xhat) * np.abs(g * xhat).mean(axis=1, keepdims=True))


def compare_quant(q_dev: np.ndarray, s_dev: np.ndarray, ref) -> Verdict:
    """Bit-exact comparison of int8 codes and float32 per-row scales."""
    q_ref, s_ref = ref
    dq = np.abs(q_dev.astype(np.int32) - q_ref.astype(np.int32))
    ds = np.asarray(s_dev, dtype=np.float32).view(np.uint32) != np.asarray(s_ref, dtype=np.float32).view(np.uint32)
    bad_q = int(np.count_nonzero(dq))
    worst = int(np.argmax(dq)) if dq.size else -1
    max_rel_s = float(np.max(np.abs(s_dev.astype(np.float64) - s_ref) / np.maximum(s_ref, 1e-300))) if s_ref.size else 0.0
    return Verdict(bad_q == 0 and not ds.any(), float(dq.max()) if dq.size else 0.0, float(bad_q),
                   max_rel_s, int(np.count_nonzero(ds)), worst)


def check_result(inp: W.HostInputs, out: dict, rows=None) -> Verdict:
    """Compare a device result {"y": ..., "row_out": ...} (host copies; the
    rows `rows` of the full result when given) with the oracle."""
    w = inp.workload
    ref = oracle_output(inp, rows=rows)
    if w.op == "quantize_int8":
        return compare_quant(out["y"], out["row_out"], ref)
    return compare(w.op, w.dtype, out["y"], ref, tolerance_scale(inp, rows))


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
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
