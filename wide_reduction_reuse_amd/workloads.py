"""Seeded synthetic inputs for the row-wise reduction-reuse operators.

This module is shared by the tests, the benchmark and the smoke check, and it
feeds both the HIP library and the CPU oracle.  It holds no operator arithmetic:
it only draws random numbers, rounds them to the storage dtype and describes the
workload shapes.

Workloads (rows x cols, distributions, seeds):

* ``softmax_f32_64x4096``     x ~ N(0, 1)                                     seed 1
* ``layernorm_bf16_4096x8192`` x = 3 N(0,1) + 0.5, gamma ~ U(0.5, 1.5),
  beta ~ N(0, 0.1), eps = 1e-5                                                seed 2
* ``rmsnorm_bf16_1024x65536`` x ~ N(0, 1), each element independently scaled by
  50 with probability 0.01; gamma ~ U(0.5, 1.5), eps = 1e-6                   seed 3
* ``softmax_f32_256x262144``  x = 4 N(0, 1) + o_row, o_row ~ U(-50, 50) per row seed 4
* the crossover sweep: {softmax, layernorm, rmsnorm} x {f32, bf16} x cols in
  {1024, 4096, 16384, 65536, 262144} x input bytes in {16 MiB, 256 MiB, 1 GiB};
  rows = bytes / (cols * element size); x ~ N(0, 1); gamma, beta, eps as above;
  seed 1000 + point index.

and the three further workloads of the CREDIT paper's evaluation (Sec. IV-A:
fp32, M = 4096 rows, 2048 for LayerNorm, widths 4096 ... 65536), at the widest
width, which the paper's traffic measurement (Fig. 5) also uses:

* ``softmax_bwd_f32_4096x65536``   logits x ~ N(0, 1), dy ~ N(0, 1)          seed 5
* ``layernorm_bwd_f32_2048x65536`` x = 3 N(0,1) + 0.5, dy ~ N(0, 1),
  gamma ~ U(0.5, 1.5), eps = 1e-5                                           seed 6
* ``quantize_int8_f32_4096x65536`` x ~ N(0, 1) with 1% of elements x50      seed 7
* the width grid of those three (``next_points``): each at cols in
  {4096, 8192, 16384, 32768, 65536}, seed 3000 + point index.

The second argument of N(mu, s) is the standard deviation.  Draw order from one
``numpy.random.Generator(PCG64(seed))``: x (float32), then the outlier mask or the
row offsets, then gamma, then beta, then dy.  bf16 values are the float32 draws
rounded to nearest, ties to even.  ``device_inputs`` draws the same
distributions on the GPU (torch's generator, same seed) for GiB-sized shapes.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

OPS = ("softmax", "layernorm", "rmsnorm", "softmax_bwd", "layernorm_bwd", "quantize_int8")
FWD_OPS = ("softmax", "layernorm", "rmsnorm")          # the crossover sweep's operators
NEXT_OPS = ("softmax_bwd", "layernorm_bwd", "quantize_int8")
DTYPES = ("f32", "bf16")
# (op, dtype) pairs with kernels: every operator in both dtypes
SUPPORTED = {(op, dt) for op in OPS for dt in DTYPES}
ELEM_BYTES = {"f32": 4, "bf16": 2}
N_PARAMS = {"softmax": 0, "layernorm": 2, "rmsnorm": 1, "softmax_bwd": 0, "layernorm_bwd": 1, "quantize_int8": 0}
N_INPUTS = {"softmax_bwd": 2, "layernorm_bwd": 2}      # row inputs per element (x, dy); others 1
ROW_OUT_BYTES = {"quantize_int8": 4}                   # fp32 scale per row
DEFAULT_EPS = {"softmax": 0.0, "layernorm": 1e-5, "rmsnorm": 1e-6, "softmax_bwd": 0.0, "layernorm_bwd": 1e-5,
               "quantize_int8": 0.0}

SWEEP_COLS = (1024, 4096, 16384, 65536, 262144)
SWEEP_BYTES = (16 << 20, 256 << 20, 1 << 30)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str
    dtype: str
    rows: int
    cols: int
    seed: int
    x_dist: str = "normal"       # normal | scaled_shifted | outliers | row_offset
    x_scale: float = 1.0
    x_shift: float = 0.0
    outlier_prob: float = 0.0
    outlier_scale: float = 1.0
    row_offset: float = 0.0      # o_row ~ U(-row_offset, row_offset)
    eps: float = 0.0

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def inputs(self) -> int:
        return N_INPUTS.get(self.op, 1)

    @property
    def out_bytes(self) -> int:
        """Bytes per output element (int8 codes for quantization)."""
        return 1 if self.op == "quantize_int8" else self.elem_bytes

    def algorithmic_bytes(self) -> int:
        """One read of every row input, one write of the output, each parameter
        vector read once and the per-row outputs written once."""
        b = self.elem_bytes
        return (self.rows * self.cols * (self.inputs * b + self.out_bytes) + self.cols * b * N_PARAMS[self.op]
                + self.rows * ROW_OUT_BYTES.get(self.op, 0))

    def with_shape(self, rows: int, cols: int, name: Optional[str] = None) -> "Workload":
        return dataclasses.replace(self, rows=rows, cols=cols, name=name or self.name)


NAMED: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("softmax_f32_64x4096", "softmax", "f32", 64, 4096, seed=1),
        Workload("layernorm_bf16_4096x8192", "layernorm", "bf16", 4096, 8192, seed=2,
                 x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5, eps=1e-5),
        Workload("rmsnorm_bf16_1024x65536", "rmsnorm", "bf16", 1024, 65536, seed=3,
                 x_dist="outliers", outlier_prob=0.01, outlier_scale=50.0, eps=1e-6),
        Workload("softmax_f32_256x262144", "softmax", "f32", 256, 262144, seed=4,
                 x_dist="row_offset", x_scale=4.0, row_offset=50.0),
        Workload("softmax_bwd_f32_4096x65536", "softmax_bwd", "f32", 4096, 65536, seed=5),
        Workload("layernorm_bwd_f32_2048x65536", "layernorm_bwd", "f32", 2048, 65536, seed=6,
                 x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5, eps=1e-5),
        Workload("quantize_int8_f32_4096x65536", "quantize_int8", "f32", 4096, 65536, seed=7,
                 x_dist="outliers", outlier_prob=0.01, outlier_scale=50.0),
        # a softmax over a vocabulary-sized odd width in bf16 (256 MiB of
        # logits): rows of odd length, held from the 4-byte word below them
        Workload("softmax_bf16_2670x50257", "softmax", "bf16", 2670, 50257, seed=8),
    ]
}
CONFIG_ORDER = ["softmax_f32_64x4096", "layernorm_bf16_4096x8192",
                "rmsnorm_bf16_1024x65536", "softmax_f32_256x262144"]
NEXT_ORDER = ["softmax_bwd_f32_4096x65536", "layernorm_bwd_f32_2048x65536", "quantize_int8_f32_4096x65536"]
EXTRA_ORDER = ["softmax_bf16_2670x50257"]
NEXT_COLS = (4096, 8192, 16384, 32768, 65536)
NEXT_ROWS = {"softmax_bwd": 4096, "layernorm_bwd": 2048, "quantize_int8": 4096}


def next_points() -> List[Workload]:
    """The paper's width grid for the three further workloads (fp32; 4096 rows,
    2048 for LayerNorm backward; the named workloads' distributions)."""
    pts = []
    idx = 0
    for name in NEXT_ORDER:
        base = NAMED[name]
        for cols in NEXT_COLS:
            rows = NEXT_ROWS[base.op]
            pts.append(dataclasses.replace(base, name="next%02d_%s_f32_%dx%d" % (idx, base.op, rows, cols),
                                           rows=rows, cols=cols, seed=3000 + idx))
            idx += 1
    return pts


OFFGRID_COLS = (3072, 12288, 24576, 49152, 98304, 196608,  # rows of whole 16-byte vectors
                1000, 5000, 30001, 50257, 100003,            # and of odd lengths
                20002)                                       # a partial last vector in both dtypes
OFFGRID_BYTES = 256 << 20


def offgrid_points() -> List[Workload]:
    """Widths off the calibration grid (which has only powers of two), where
    the selector prices plans with its analytic model: the forward operators,
    both dtypes, 256 MiB of input."""
    pts = []
    idx = 0
    for op in FWD_OPS:
        for dt in DTYPES:
            for cols in OFFGRID_COLS:
                rows = OFFGRID_BYTES // (cols * ELEM_BYTES[dt])
                pts.append(Workload("offgrid%02d_%s_%s_%dx%d" % (idx, op, dt, rows, cols), op, dt, rows, cols,
                                    seed=5000 + idx, eps=DEFAULT_EPS[op]))
                idx += 1
    return pts


# Widths around the LDS tier's reach (256 MiB of input each): the widest row
# registers alone hold on path 1, and wider ones up to what registers plus
# 128 KiB of LDS hold (one input: 65536 -> 98304 fp32, 131072 -> 196608 bf16;
# two inputs: 32768 -> 49152 fp32 and 65536 -> 98304 bf16).
LDS_COLS = {("f32", 1): (49152, 65536, 81920, 98304), ("bf16", 1): (98304, 131072, 163840, 196608),
            ("f32", 2): (32768, 40960, 49152), ("bf16", 2): (65536, 81920, 98304)}
LDS_BYTES = 256 << 20


def lds_points() -> List[Workload]:
    """Every operator and dtype at the widths where the LDS tier decides
    whether one owner can hold a row (LDS_COLS)."""
    pts = []
    idx = 0
    for op in OPS:
        for dt in DTYPES:
            if (op, dt) not in SUPPORTED:
                continue
            for cols in LDS_COLS[(dt, 2 if op in ("softmax_bwd", "layernorm_bwd") else 1)]:
                rows = LDS_BYTES // (cols * ELEM_BYTES[dt])
                pts.append(Workload("lds%02d_%s_%s_%dx%d" % (idx, op, dt, rows, cols), op, dt, rows, cols,
                                    seed=7000 + idx, eps=DEFAULT_EPS[op]))
                idx += 1
    return pts


CALIB_BYTES = (8 << 20, 64 << 20, 512 << 20, 2048 << 20)
CALIB_COLS = tuple(1 << k for k in range(10, 19))  # 1024 ... 262144


def calibration_points() -> List[Workload]:
    """The selector's calibration shapes: the sweep's operators and dtypes at
    every power-of-two width from 1024 to 262144, at input sizes the scored
    sweep does not use (8, 64, 512 and 2048 MiB, bracketing its 16 MiB,
    256 MiB and 1 GiB)."""
    pts = []
    idx = 0
    for op in FWD_OPS:
        for dt in DTYPES:
            for cols in CALIB_COLS:
                for nbytes in CALIB_BYTES:
                    rows = nbytes // (cols * ELEM_BYTES[dt])
                    name = "calib%02d_%s_%s_%dx%d" % (idx, op, dt, rows, cols)
                    pts.append(Workload(name, op, dt, rows, cols, seed=2000 + idx, eps=DEFAULT_EPS[op]))
                    idx += 1
    return pts


# Widths between the powers of two, near 2^(k + 1/2): whole 16-byte vectors
# (multiples of 256 elements) and odd lengths.  With them a tile, which is
# timed only where it is at least half used, has measured widths on both sides
# of most widths off the grid.
CALIB_MID_COLS = tuple(round(2 ** (k + 0.5) / 256) * 256 for k in range(10, 18))  # 1536 ... 185344
CALIB_ODD_COLS = tuple((1 << k) + 1 for k in (10, 12, 14, 16, 17, 18))  # 1025 ... 262145
CALIB_ODD_MID_COLS = tuple(round(2 ** (k + 0.5)) | 1 for k in (10, 12, 14, 15, 16, 17))  # 1449 ... 185365
# Even bf16 widths that are not multiples of 8 elements: their rows end in a
# partial 16-byte vector (the fp32 rows of the odd widths above do too).
CALIB_PART_COLS = (tuple((1 << k) + 2 for k in (10, 12, 14, 16, 17, 18)) +                       # 1026 ... 262146
                   tuple(round(2 ** (k + 0.5)) // 8 * 8 + 2 for k in (10, 12, 14, 15, 16, 17)))  # 1450 ... 185362


def calibration_points_mid() -> List[Workload]:
    """Calibration shapes at the aligned widths between the powers of two
    (CALIB_MID_COLS), the forward operators, both dtypes, the sizes of
    calibration_points()."""
    pts = []
    idx = 0
    for op in FWD_OPS:
        for dt in DTYPES:
            for cols in CALIB_MID_COLS:
                for nbytes in CALIB_BYTES:
                    rows = max(1, nbytes // (cols * ELEM_BYTES[dt]))
                    pts.append(Workload("calibm%03d_%s_%s_%dx%d" % (idx, op, dt, rows, cols), op, dt, rows, cols,
                                        seed=7000 + idx, eps=DEFAULT_EPS[op]))
                    idx += 1
    return pts


def calibration_points_odd() -> List[Workload]:
    """Calibration shapes for rows that are not whole 16-byte vectors (their
    kernels use 4- or 2-byte accesses and tiles of their own): the forward
    operators, both dtypes, widths 2^k + 1 and odd widths near 2^(k + 1/2),
    at the sizes of calibration_points()."""
    pts = []
    idx = 0
    for op in FWD_OPS:
        for dt in DTYPES:
            for cols in CALIB_ODD_COLS + CALIB_ODD_MID_COLS:
                for nbytes in CALIB_BYTES:
                    rows = max(1, nbytes // (cols * ELEM_BYTES[dt]))
                    pts.append(Workload("calibo%03d_%s_%s_%dx%d" % (idx, op, dt, rows, cols), op, dt, rows, cols,
                                        seed=6000 + idx, eps=DEFAULT_EPS[op]))
                    idx += 1
    return pts


def calibration_points_part() -> List[Workload]:
    """Calibration shapes for bf16 rows that end in a partial 16-byte vector
    (CALIB_PART_COLS): the forward operators at the sizes of
    calibration_points(), softmax backward at the rows of
    calibration_points_next()."""
    pts = []
    idx = 0
    for op in FWD_OPS:
        for cols in CALIB_PART_COLS:
            for nbytes in CALIB_BYTES:
                rows = max(1, nbytes // (cols * ELEM_BYTES["bf16"]))
                pts.append(Workload("calibp%03d_%s_bf16_%dx%d" % (idx, op, rows, cols), op, "bf16", rows, cols,
                                    seed=9000 + idx, eps=DEFAULT_EPS[op]))
                idx += 1
    base = NAMED["softmax_bwd_f32_4096x65536"]
    for cols in CALIB_PART_COLS:
        for rows in CALIB_NEXT_ROWS:
            if rows * cols * ELEM_BYTES["bf16"] <= CALIB_NEXT_MAX_BYTES:
                pts.append(dataclasses.replace(
                    base, name="calibp%03d_softmax_bwd_bf16_%dx%d" % (idx, rows, cols), dtype="bf16",
                    rows=rows, cols=cols, seed=9000 + idx))
                idx += 1
    return pts


CALIB_NEXT_ROWS = (512, 1536, 6144, 16384)
CALIB_NEXT_MAX_BYTES = 4 << 30  # of x


def calibration_points_next() -> List[Workload]:
    """Calibration shapes of the three further workloads: each supported dtype
    at every power-of-two width from 1024 to 262144, at row counts that bracket
    (and never equal) the 2048 and 4096 rows of their width grid, x at most
    4 GiB."""
    pts = []
    idx = 0
    for name in NEXT_ORDER:
        base = NAMED[name]
        for dt in DTYPES:
            if (base.op, dt) not in SUPPORTED:
                continue
            for cols in CALIB_COLS:
                for rows in CALIB_NEXT_ROWS:
                    if rows * cols * ELEM_BYTES[dt] > CALIB_NEXT_MAX_BYTES:
                        continue
                    pts.append(dataclasses.replace(
                        base, name="calibn%03d_%s_%s_%dx%d" % (idx, base.op, dt, rows, cols), dtype=dt,
                        rows=rows, cols=cols, seed=4000 + idx))
                    idx += 1
    return pts


def calibration_points_next_more() -> List[Workload]:
    """The further workloads' calibration at the widths between the powers of
    two and the odd widths (CALIB_MID_COLS, CALIB_ODD_COLS,
    CALIB_ODD_MID_COLS), at the rows of calibration_points_next()."""
    pts = []
    idx = 0
    for name in NEXT_ORDER:
        base = NAMED[name]
        for dt in DTYPES:
            if (base.op, dt) not in SUPPORTED:
                continue
            for cols in CALIB_MID_COLS + CALIB_ODD_COLS + CALIB_ODD_MID_COLS:
                for rows in CALIB_NEXT_ROWS:
                    if rows * cols * ELEM_BYTES[dt] > CALIB_NEXT_MAX_BYTES:
                        continue
                    pts.append(dataclasses.replace(
                        base, name="calibx%03d_%s_%s_%dx%d" % (idx, base.op, dt, rows, cols), dtype=dt,
                        rows=rows, cols=cols, seed=8000 + idx))
                    idx += 1
    return pts


def offgrid_points_next() -> List[Workload]:
    """The further workloads at the off-grid widths (OFFGRID_COLS), each
    supported dtype, at the rows of their width grid (4096; 2048 for
    LayerNorm backward)."""
    pts = []
    idx = 0
    for name in NEXT_ORDER:
        base = NAMED[name]
        for dt in DTYPES:
            if (base.op, dt) not in SUPPORTED:
                continue
            for cols in OFFGRID_COLS:
                rows = NEXT_ROWS[base.op]
                pts.append(dataclasses.replace(
                    base, name="offgridn%02d_%s_%s_%dx%d" % (idx, base.op, dt, rows, cols), dtype=dt,
                    rows=rows, cols=cols, seed=9000 + idx))
                idx += 1
    return pts


def sweep_points() -> List[Workload]:
    """The 90-point crossover sweep, in a fixed order (op, dtype, cols, bytes)."""
    pts = []
    idx = 0
    for op in FWD_OPS:
        for dt in DTYPES:
            for cols in SWEEP_COLS:
                for nbytes in SWEEP_BYTES:
                    rows = nbytes // (cols * ELEM_BYTES[dt])
                    name = "sweep%02d_%s_%s_%dx%d" % (idx, op, dt, rows, cols)
                    pts.append(Workload(name, op, dt, rows, cols, seed=1000 + idx,
                                        eps=DEFAULT_EPS[op]))
                    idx += 1
    return pts


# ---------------------------------------------------------------------------
# rounding of the generated float32 draws to the bf16 storage type
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, nearest-even (inputs are finite draws)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class HostInputs:
    """Generated inputs in storage form: float32 arrays, or uint16 bf16 bit patterns."""
    workload: Workload
    x: np.ndarray
    gamma: Optional[np.ndarray]
    beta: Optional[np.ndarray]
    eps: float
    dy: Optional[np.ndarray] = None


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def generate(w: Workload) -> HostInputs:
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.rows, w.cols)
    x = rng.standard_normal(shape, dtype=np.float32)
    if w.x_dist == "scaled_shifted":
        x *= np.float32(w.x_scale)
        x += np.float32(w.x_shift)
    elif w.x_dist == "outliers":
        mask = rng.random(shape, dtype=np.float32) < np.float32(w.outlier_prob)
        x[mask] *= np.float32(w.outlier_scale)
    elif w.x_dist == "row_offset":
        off = rng.uniform(-w.row_offset, w.row_offset, size=(w.rows, 1)).astype(np.float32)
        x *= np.float32(w.x_scale)
        x += off
    elif w.x_dist != "normal":
        raise ValueError("unknown x_dist %r" % w.x_dist)
    gamma = beta = dy = None
    if N_PARAMS[w.op] >= 1:
        gamma = rng.uniform(0.5, 1.5, size=w.cols).astype(np.float32)
    if N_PARAMS[w.op] >= 2:
        beta = (rng.standard_normal(w.cols, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    if w.inputs >= 2:
        dy = rng.standard_normal(shape, dtype=np.float32)
    return HostInputs(w, _store(x, w.dtype),
                      None if gamma is None else _store(gamma, w.dtype),
                      None if beta is None else _store(beta, w.dtype),
                      float(np.float32(w.eps)),
                      None if dy is None else _store(dy, w.dtype))


# ---------------------------------------------------------------------------
# device copies (torch is imported only here)
# ---------------------------------------------------------------------------
def to_device(inp: HostInputs) -> dict:
    """The inputs as device tensors: {x, dy, gamma, beta} (absent ones None)."""
    import torch

    def dev(a):
        if a is None:
            return None
        if inp.workload.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()
    return {"x": dev(inp.x), "dy": dev(inp.dy), "gamma": dev(inp.gamma), "beta": dev(inp.beta)}


def alloc_outputs(w: Workload, t: dict) -> dict:
    """Adds the output tensors y (int8 codes for quantization) and row_out
    (the per-row scale, quantization only) to the operand mapping t."""
    import torch
    x = t["x"]
    if w.op == "quantize_int8":
        t["y"] = torch.empty(x.shape, dtype=torch.int8, device=x.device)
        t["row_out"] = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    else:
        t["y"] = torch.empty_like(x)
        t["row_out"] = None
    return t


def device_inputs(w: Workload) -> dict:
    """The operand mapping of w with its inputs drawn on the device, for
    GiB-sized shapes that need no host-side generation: x (and dy, gamma,
    beta) from w's distributions with torch's generator seeded with w.seed,
    drawn in float32 and rounded to the storage dtype (bf16: nearest, ties to
    even); outputs allocated (alloc_outputs).  The values differ from
    generate()'s (another generator); a check copies the rows it compares,
    and the parameters, to the host."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    x = torch.randn((w.rows, w.cols), generator=g, device="cuda", dtype=torch.float32)
    if w.x_dist == "scaled_shifted":
        x.mul_(w.x_scale).add_(w.x_shift)
    elif w.x_dist == "outliers":
        mask = torch.rand((w.rows, w.cols), generator=g, device="cuda") < w.outlier_prob
        x = torch.where(mask, x * w.outlier_scale, x)
    elif w.x_dist == "row_offset":
        off = (torch.rand((w.rows, 1), generator=g, device="cuda") * 2.0 - 1.0) * w.row_offset
        x.mul_(w.x_scale).add_(off)
    elif w.x_dist != "normal":
        raise ValueError("unknown x_dist %r" % w.x_dist)
    gamma = beta = dy = None
    if N_PARAMS[w.op] >= 1:
        gamma = torch.rand(w.cols, generator=g, device="cuda") + 0.5
    if N_PARAMS[w.op] >= 2:
        beta = torch.randn(w.cols, generator=g, device="cuda") * 0.1
    if w.inputs >= 2:
        dy = torch.randn((w.rows, w.cols), generator=g, device="cuda", dtype=torch.float32)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    cast = (lambda t: None if t is None else t.to(dt).contiguous())
    return alloc_outputs(w, {"x": cast(x), "dy": cast(dy), "gamma": cast(gamma), "beta": cast(beta)})


def custom(op: str, dtype: str, rows: int, cols: int, seed: int, **kw) -> Workload:
    eps = kw.pop("eps", DEFAULT_EPS[op])
    return Workload("%s_%s_%dx%d_s%d" % (op, dtype, rows, cols, seed), op, dtype, rows, cols,
                    seed=seed, eps=eps, **kw)
