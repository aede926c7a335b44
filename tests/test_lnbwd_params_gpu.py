"""LayerNorm backward's statistics output and parameter gradients on the GPU
against the oracle.

The row part writes each row's (mean, rstd) when asked
(credit_layernorm_backward_stats); the parameter part sums dy * xhat and dy
over the rows (credit_layernorm_backward_params).  Tolerances, for fp32
arithmetic on either dtype's inputs:
  * mean_i within 1e-5 of the row's root mean square, rstd_i within 1e-5
    relative;
  * dgamma_j within 1e-5 * sum_i |dy_ij| (|x_ij| + m_i) rstd_i, m_i the row's
    root mean square, and dbeta_j within 1e-5 * sum_i |dy_ij| of the oracle:
    the rounding error of a sum is bounded in proportion to the sum of its
    terms' magnitudes (terms of both signs may cancel), and each term's
    xhat_ij = (x_ij - mean_i) rstd_i is a difference whose fp32 error scales
    with |x_ij| and the row's size, not with xhat_ij (which is near zero
    where x_ij is near the mean).
Shapes: the 2048 x 65536 fp32 workload, smaller ones with ragged column
blocks and row groups, rows whose byte length is not a multiple of 16 bytes
(element accesses), one row, no rows.  bf16 inputs take their statistics
from the oracle (the bf16 row part is tested with the other operators).
"""
import numpy as np
import pytest

import oracle
from wide_reduction_reuse_amd import workloads as W

from parity import host_values, to_device

pytestmark = pytest.mark.gpu


def _lib():
    import torch
    from wide_reduction_reuse_amd import credit
    assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
    return credit


def _inputs(dt, rows, cols, seed):
    w = W.custom("layernorm_bwd", dt, rows, cols, seed=seed, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    return inp, host_values(inp.x, dt), host_values(inp.dy, dt)


def _check_params(x, dy, eps, dg, db, label):
    ref_g, ref_b = oracle.layernorm_backward_params(x, dy, eps)
    mu, rstd = oracle.layernorm_row_stats(x, eps)
    rms = np.sqrt((x * x).mean(axis=1))
    mag_g = (np.abs(dy) * (np.abs(x) + rms[:, None]) * rstd[:, None]).sum(axis=0)
    mag_b = np.abs(dy).sum(axis=0)
    eg = np.abs(dg - ref_g) / np.maximum(mag_g, 1e-30)
    eb = np.abs(db - ref_b) / np.maximum(mag_b, 1e-30)
    print("%s: dgamma err %.3g, dbeta err %.3g (of the summed magnitudes)" % (label, eg.max(initial=0),
                                                                               eb.max(initial=0)), flush=True)
    assert (eg <= 1e-5).all(), (label, int(np.argmax(eg)), eg.max())
    assert (eb <= 1e-5).all(), (label, int(np.argmax(eb)), eb.max())


@pytest.mark.parametrize("rows,cols", [(2048, 65536), (37, 4096), (300, 20480), (1, 1000), (5, 30001),
                                       (300, 20002), (9, 3), (4100, 1024)])
def test_stats_and_params_fp32(rows, cols):
    import torch
    C = _lib()
    inp, x, dy = _inputs("f32", rows, cols, seed=rows * 7 + cols)
    eps = inp.eps
    xd, dyd, gd = (to_device(a, "f32") for a in (inp.x, inp.dy, inp.gamma))
    dx, stats = C.credit_layernorm_backward_stats(xd, dyd, gd, eps)
    dg, db = C.credit_layernorm_backward_params(xd, dyd, stats)
    torch.cuda.synchronize()
    C.credit_check_errors()
    st = stats.cpu().numpy().astype(np.float64)
    mu, rstd = oracle.layernorm_row_stats(x, eps)
    rms = np.sqrt((x * x).mean(axis=1))
    assert (np.abs(st[:, 0] - mu) <= 1e-5 * rms).all()
    assert (np.abs(st[:, 1] - rstd) <= 1e-5 * rstd).all()
    # the row part is unchanged by writing the statistics
    ref_dx = oracle.layernorm_backward(x, dy, host_values(inp.gamma, "f32"), eps)
    dx0 = C.credit_layernorm_backward(xd, dyd, gd, eps)
    torch.cuda.synchronize()
    assert np.array_equal(dx.cpu().numpy(), dx0.cpu().numpy())
    assert np.isfinite(ref_dx).all()
    _check_params(x, dy, eps, dg.cpu().numpy().astype(np.float64), db.cpu().numpy().astype(np.float64),
                  "fp32 %dx%d" % (rows, cols))


@pytest.mark.parametrize("rows,cols", [(2048, 8192), (37, 50257), (100, 4096), (3, 20002)])
def test_params_bf16_inputs(rows, cols):
    import torch
    C = _lib()
    inp, x, dy = _inputs("bf16", rows, cols, seed=rows * 5 + cols)
    mu, rstd = oracle.layernorm_row_stats(x, inp.eps)
    stats = torch.tensor(np.stack([mu, rstd], axis=1).astype(np.float32), device="cuda")
    dg, db = C.credit_layernorm_backward_params(to_device(inp.x, "bf16"), to_device(inp.dy, "bf16"), stats)
    torch.cuda.synchronize()
    _check_params(x, dy, inp.eps, dg.cpu().numpy().astype(np.float64), db.cpu().numpy().astype(np.float64),
                  "bf16 %dx%d" % (rows, cols))


def test_params_no_rows_and_errors():
    import torch
    C = _lib()
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    st = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    dg, db = C.credit_layernorm_backward_params(x, x, st)
    torch.cuda.synchronize()
    assert not dg.any() and not db.any()
    L = C.lib()
    import ctypes
    p = ctypes.c_void_p(x.data_ptr() if x.numel() else 256)
    # too small a workspace, for a shape that needs one
    xs = torch.zeros((64, 64), device="cuda")
    st = torch.zeros((64, 2), device="cuda")
    out = torch.zeros(64, device="cuda")
    assert L.credit_layernorm_backward_params(ctypes.c_void_p(xs.data_ptr()), ctypes.c_void_p(xs.data_ptr()),
                                              ctypes.c_void_p(st.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                              ctypes.c_void_p(out.data_ptr()), 64, 64, 0, p, 16, None) == 1
