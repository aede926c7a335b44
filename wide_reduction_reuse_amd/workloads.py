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

The second argument of N(mu, s) is the standard deviation.  Draw order from one
``numpy.random.Generator(PCG64(seed))``: x (float32), then the outlier mask or the
row offsets, then gamma, then beta.  bf16 values are the float32 draws rounded to
nearest, ties to even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

OPS = ("softmax", "layernorm", "rmsnorm")
DTYPES = ("f32", "bf16")
ELEM_BYTES = {"f32": 4, "bf16": 2}
N_PARAMS = {"softmax": 0, "layernorm": 2, "rmsnorm": 1}
DEFAULT_EPS = {"softmax": 0.0, "layernorm": 1e-5, "rmsnorm": 1e-6}

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

    def algorithmic_bytes(self) -> int:
        """One read of x, one write of y, and each parameter vector read once."""
        b = self.elem_bytes
        return self.rows * self.cols * 2 * b + self.cols * b * N_PARAMS[self.op]

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
    ]
}
CONFIG_ORDER = ["softmax_f32_64x4096", "layernorm_bf16_4096x8192",
                "rmsnorm_bf16_1024x65536", "softmax_f32_256x262144"]


CALIB_BYTES = (8 << 20, 64 << 20, 512 << 20, 2048 << 20)
CALIB_COLS = tuple(1 << k for k in range(10, 19))  # 1024 ... 262144


def calibration_points() -> List[Workload]:
    """The selector's calibration shapes: the sweep's operators and dtypes at
    every power-of-two width from 1024 to 262144, at input sizes the scored
    sweep does not use (8, 64, 512 and 2048 MiB, bracketing its 16 MiB,
    256 MiB and 1 GiB)."""
    pts = []
    idx = 0
    for op in OPS:
        for dt in DTYPES:
            for cols in CALIB_COLS:
                for nbytes in CALIB_BYTES:
                    rows = nbytes // (cols * ELEM_BYTES[dt])
                    name = "calib%02d_%s_%s_%dx%d" % (idx, op, dt, rows, cols)
                    pts.append(Workload(name, op, dt, rows, cols, seed=2000 + idx, eps=DEFAULT_EPS[op]))
                    idx += 1
    return pts


def sweep_points() -> List[Workload]:
    """The 90-point crossover sweep, in a fixed order (op, dtype, cols, bytes)."""
    pts = []
    idx = 0
    for op in OPS:
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
    gamma = beta = None
    if w.op in ("layernorm", "rmsnorm"):
        gamma = rng.uniform(0.5, 1.5, size=w.cols).astype(np.float32)
    if w.op == "layernorm":
        beta = (rng.standard_normal(w.cols, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return HostInputs(w, _store(x, w.dtype),
                      None if gamma is None else _store(gamma, w.dtype),
                      None if beta is None else _store(beta, w.dtype),
                      float(np.float32(w.eps)))


def custom(op: str, dtype: str, rows: int, cols: int, seed: int, **kw) -> Workload:
    eps = kw.pop("eps", DEFAULT_EPS[op])
    return Workload("%s_%s_%dx%d_s%d" % (op, dtype, rows, cols, seed), op, dtype, rows, cols,
                    seed=seed, eps=eps, **kw)
