"""Double-precision CPU oracle for the row-wise reduction-reuse operators.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library (``wide_reduction_reuse_amd``) and never calls it.

The arithmetic lives in ``oracle.c`` (plain C, double, OpenMP over rows); this
module only builds that file with gcc, loads it with ctypes and converts inputs
to float64 exactly.  Operator definitions and the readings taken where the
CREDIT paper is silent are stated at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_softmax.argtypes = [_D, _D, _I64, _I64]
        lib.oracle_layernorm.argtypes = [_D, _D, _D, ctypes.c_double, _D, _I64, _I64]
        lib.oracle_rmsnorm.argtypes = [_D, _D, ctypes.c_double, _D, _I64, _I64]
        lib.oracle_softmax_stats.argtypes = [_D, _I64, _I64, _D, _D]
        lib.oracle_layernorm_stats.argtypes = [_D, _I64, _I64, _D, _D]
        P64 = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_softmax_partials.argtypes = [_D, P64, ctypes.c_int, _D, _D]
        lib.oracle_softmax_merge.argtypes = [_D, _D, ctypes.c_int, _D, _D]
        lib.oracle_layernorm_partials.argtypes = [_D, P64, ctypes.c_int, _D, _D, _D]
        lib.oracle_layernorm_merge.argtypes = [_D, _D, _D, ctypes.c_int, _D, _D, _D]
        lib.oracle_rmsnorm_partials.argtypes = [_D, P64, ctypes.c_int, _D]
        lib.oracle_round_bf16.argtypes = [_D, ctypes.POINTER(ctypes.c_uint16), _I64]
        lib.oracle_softmax_backward.argtypes = [_D, _D, _D, _I64, _I64]
        lib.oracle_layernorm_backward.argtypes = [_D, _D, _D, ctypes.c_double, _D, _I64, _I64]
        lib.oracle_layernorm_row_stats.argtypes = [_D, ctypes.c_double, _D, _D, _I64, _I64]
        lib.oracle_layernorm_backward_params.argtypes = [_D, _D, _D, _D, _D, _D, _I64, _I64]
        lib.oracle_quantize_int8.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int8),
                                             ctypes.POINTER(ctypes.c_float), _I64, _I64]
        lib.oracle_softmax_backward_stats.argtypes = [_D, _D, _I64, _I64, _D, _D, _D]
        lib.oracle_softmax_backward_partials.argtypes = [_D, _D, P64, ctypes.c_int, _D, _D, _D]
        lib.oracle_softmax_backward_merge.argtypes = [_D, _D, _D, ctypes.c_int, _D, _D, _D]
        lib.oracle_layernorm_backward_stats.argtypes = [_D, _D, _I64, _I64, _D, _D, _D, _D]
        lib.oracle_layernorm_backward_partials.argtypes = [_D, _D, P64, ctypes.c_int, _D, _D, _D, _D, _D]
        lib.oracle_layernorm_backward_merge.argtypes = [_D, _D, _D, _D, _D, ctypes.c_int, _D, _D, _D, _D, _D]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(_D)


def _as_f64_2d(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.ndim == 1:
        a = a.reshape(1, -1)
    if a.ndim != 2:
        raise ValueError("expected a 2-D [rows, cols] array")
    return a


def _as_f64_1d(v, n: int) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(-1))
    if a.shape[0] != n:
        raise ValueError("parameter vector length %d != cols %d" % (a.shape[0], n))
    return a


# ---------------------------------------------------------------------------
# exact input decoding (bf16 bit patterns -> float64)
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the pattern is the top half of a float."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# operators
# ---------------------------------------------------------------------------
def softmax(x) -> np.ndarray:
    a = _as_f64_2d(x)
    y = np.empty_like(a)
    if a.size:
        _load().oracle_softmax(_dptr(a), _dptr(y), a.shape[0], a.shape[1])
    return y


def layernorm(x, gamma, beta, eps: float) -> np.ndarray:
    a = _as_f64_2d(x)
    g = _as_f64_1d(gamma, a.shape[1])
    b = _as_f64_1d(beta, a.shape[1])
    y = np.empty_like(a)
    if a.size:
        _load().oracle_layernorm(_dptr(a), _dptr(g), _dptr(b), float(eps), _dptr(y),
                                 a.shape[0], a.shape[1])
    return y


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    a = _as_f64_2d(x)
    g = _as_f64_1d(gamma, a.shape[1])
    y = np.empty_like(a)
    if a.size:
        _load().oracle_rmsnorm(_dptr(a), _dptr(g), float(eps), _dptr(y), a.shape[0], a.shape[1])
    return y


def softmax_stats(x):
    a = _as_f64_2d(x)
    m = np.empty(a.shape[0])
    s = np.empty(a.shape[0])
    _load().oracle_softmax_stats(_dptr(a), a.shape[0], a.shape[1], _dptr(m), _dptr(s))
    return m, s


def layernorm_stats(x):
    a = _as_f64_2d(x)
    mu = np.empty(a.shape[0])
    m2 = np.empty(a.shape[0])
    _load().oracle_layernorm_stats(_dptr(a), a.shape[0], a.shape[1], _dptr(mu), _dptr(m2))
    return mu, m2


def _bounds(bounds, n: int) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bounds, dtype=np.int64))
    if b[0] != 0 or b[-1] != n or np.any(np.diff(b) < 0):
        raise ValueError("bounds must run from 0 to cols and be non-decreasing")
    return b


def softmax_partials(xrow, bounds):
    x = np.ascontiguousarray(np.asarray(xrow, dtype=np.float64))
    b = _bounds(bounds, x.shape[0])
    p = b.shape[0] - 1
    m = np.empty(p)
    s = np.empty(p)
    _load().oracle_softmax_partials(_dptr(x), b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    p, _dptr(m), _dptr(s))
    return m, s


def softmax_merge(m_c, s_c):
    m_c = np.ascontiguousarray(m_c, dtype=np.float64)
    s_c = np.ascontiguousarray(s_c, dtype=np.float64)
    m = ctypes.c_double()
    s = ctypes.c_double()
    _load().oracle_softmax_merge(_dptr(m_c), _dptr(s_c), m_c.shape[0], ctypes.byref(m), ctypes.byref(s))
    return m.value, s.value


def layernorm_partials(xrow, bounds):
    x = np.ascontiguousarray(np.asarray(xrow, dtype=np.float64))
    b = _bounds(bounds, x.shape[0])
    p = b.shape[0] - 1
    n = np.empty(p)
    mu = np.empty(p)
    m2 = np.empty(p)
    _load().oracle_layernorm_partials(_dptr(x), b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      p, _dptr(n), _dptr(mu), _dptr(m2))
    return n, mu, m2


def layernorm_merge(n_c, mu_c, m2_c):
    n_c = np.ascontiguousarray(n_c, dtype=np.float64)
    mu_c = np.ascontiguousarray(mu_c, dtype=np.float64)
    m2_c = np.ascontiguousarray(m2_c, dtype=np.float64)
    n = ctypes.c_double()
    mu = ctypes.c_double()
    m2 = ctypes.c_double()
    _load().oracle_layernorm_merge(_dptr(n_c), _dptr(mu_c), _dptr(m2_c), n_c.shape[0],
                                   ctypes.byref(n), ctypes.byref(mu), ctypes.byref(m2))
    return n.value, mu.value, m2.value


def rmsnorm_partials(xrow, bounds):
    x = np.ascontiguousarray(np.asarray(xrow, dtype=np.float64))
    b = _bounds(bounds, x.shape[0])
    p = b.shape[0] - 1
    ss = np.empty(p)
    _load().oracle_rmsnorm_partials(_dptr(x), b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    p, _dptr(ss))
    return ss


def round_bf16(y) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even), returned as uint16 bits."""
    a = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    if a.size:
        _load().oracle_round_bf16(_dptr(a), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), a.size)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# the three further workloads (definitions and readings at the end of oracle.c)
# ---------------------------------------------------------------------------
def softmax_backward(x, dy) -> np.ndarray:
    """Gradient of row-wise softmax with respect to its logits x, given dy."""
    a = _as_f64_2d(x)
    g = _as_f64_2d(dy)
    if g.shape != a.shape:
        raise ValueError("dy must have x's shape")
    out = np.empty_like(a)
    if a.size:
        _load().oracle_softmax_backward(_dptr(a), _dptr(g), _dptr(out), a.shape[0], a.shape[1])
    return out


def layernorm_backward(x, dy, gamma, eps: float) -> np.ndarray:
    """Row part of the LayerNorm gradient: dL/dx given dL/dy (statistics recomputed from x)."""
    a = _as_f64_2d(x)
    g = _as_f64_2d(dy)
    if g.shape != a.shape:
        raise ValueError("dy must have x's shape")
    gam = _as_f64_1d(gamma, a.shape[1])
    out = np.empty_like(a)
    if a.size:
        _load().oracle_layernorm_backward(_dptr(a), _dptr(g), _dptr(gam), float(eps), _dptr(out),
                                          a.shape[0], a.shape[1])
    return out


def layernorm_row_stats(x, eps: float):
    """Per-row mean and 1 / sqrt(biased variance + eps) of x [rows][cols]."""
    a = _as_f64_2d(x)
    rows, cols = a.shape
    mu = np.empty(rows)
    rstd = np.empty(rows)
    if rows:
        _load().oracle_layernorm_row_stats(_dptr(a), float(eps), _dptr(mu), _dptr(rstd), rows, cols)
    return mu, rstd


def layernorm_backward_params(x, dy, eps: float):
    """LayerNorm backward, parameter part: (dgamma, dbeta) [cols], sums over the
    rows of dy * xhat and of dy."""
    a = _as_f64_2d(x)
    g = _as_f64_2d(dy)
    rows, cols = a.shape
    mu, rstd = layernorm_row_stats(a, eps)
    dgam = np.zeros(cols)
    dbet = np.zeros(cols)
    if rows and cols:
        _load().oracle_layernorm_backward_params(_dptr(a), _dptr(g), _dptr(mu), _dptr(rstd), _dptr(dgam),
                                                 _dptr(dbet), rows, cols)
    return dgam, dbet


def quantize_int8(x):
    """Row-wise symmetric int8 quantization of float32 values: (codes int8 [rows, cols],
    scale float32 [rows]), computed in IEEE single precision."""
    a = np.asarray(x)
    if a.dtype != np.float32:
        raise TypeError("quantize_int8 takes float32 values (decode bf16 with bf16_bits_to_f32)")
    a = np.ascontiguousarray(a)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    if a.ndim != 2:
        raise ValueError("expected a 2-D [rows, cols] array")
    q = np.empty(a.shape, dtype=np.int8)
    scale = np.empty(a.shape[0], dtype=np.float32)
    if a.size:
        _load().oracle_quantize_int8(a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                     q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)),
                                     scale.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), a.shape[0], a.shape[1])
    return q, scale


def softmax_backward_stats(x, dy):
    a = _as_f64_2d(x)
    g = _as_f64_2d(dy)
    m, s, u = (np.empty(a.shape[0]) for _ in range(3))
    _load().oracle_softmax_backward_stats(_dptr(a), _dptr(g), a.shape[0], a.shape[1], _dptr(m), _dptr(s), _dptr(u))
    return m, s, u


def softmax_backward_partials(xrow, dyrow, bounds):
    x = np.ascontiguousarray(np.asarray(xrow, dtype=np.float64))
    g = np.ascontiguousarray(np.asarray(dyrow, dtype=np.float64))
    b = _bounds(bounds, x.shape[0])
    p = b.shape[0] - 1
    m, s, u = (np.empty(p) for _ in range(3))
    _load().oracle_softmax_backward_partials(_dptr(x), _dptr(g), b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                             p, _dptr(m), _dptr(s), _dptr(u))
    return m, s, u


def softmax_backward_merge(m_c, s_c, u_c):
    m_c, s_c, u_c = (np.ascontiguousarray(v, dtype=np.float64) for v in (m_c, s_c, u_c))
    out = [ctypes.c_double() for _ in range(3)]
    _load().oracle_softmax_backward_merge(_dptr(m_c), _dptr(s_c), _dptr(u_c), m_c.shape[0],
                                          *(ctypes.byref(o) for o in out))
    return tuple(o.value for o in out)


def layernorm_backward_stats(x, g):
    """Per row: (mean, M2, sum g, sum g (x - mean)) for g = gamma * dy given directly."""
    a = _as_f64_2d(x)
    gg = _as_f64_2d(g)
    mu, m2, sa, sb = (np.empty(a.shape[0]) for _ in range(4))
    _load().oracle_layernorm_backward_stats(_dptr(a), _dptr(gg), a.shape[0], a.shape[1], _dptr(mu), _dptr(m2),
                                            _dptr(sa), _dptr(sb))
    return mu, m2, sa, sb


def layernorm_backward_partials(xrow, grow, bounds):
    x = np.ascontiguousarray(np.asarray(xrow, dtype=np.float64))
    g = np.ascontiguousarray(np.asarray(grow, dtype=np.float64))
    b = _bounds(bounds, x.shape[0])
    p = b.shape[0] - 1
    outs = [np.empty(p) for _ in range(5)]
    _load().oracle_layernorm_backward_partials(_dptr(x), _dptr(g), b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                               p, *(_dptr(o) for o in outs))
    return tuple(outs)


def layernorm_backward_merge(n_c, mu_c, m2_c, a_c, b_c):
    ins = [np.ascontiguousarray(v, dtype=np.float64) for v in (n_c, mu_c, m2_c, a_c, b_c)]
    out = [ctypes.c_double() for _ in range(5)]
    _load().oracle_layernorm_backward_merge(*(_dptr(v) for v in ins), ins[0].shape[0],
                                            *(ctypes.byref(o) for o in out))
    return tuple(o.value for o in out)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))
