"""Pins for the oracle of LayerNorm backward's parameter part, the gradients
with respect to gamma and beta (the column sums of the LayerNorm workload of
the CREDIT paper's evaluation, Sec. IV-A).

Pinned to torch's float64 autograd of layer_norm (a library routine), to
finite differences of the already pinned forward LayerNorm oracle (the loss
sum(dy * y) is linear in gamma and beta, so a unit step gives the gradient
up to rounding), to the per-row statistics from numpy, and to closed forms:
one row, a constant dy, dy = xhat."""
import numpy as np
import pytest
import torch

import oracle


def _rand(rows, cols, seed, scale=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols)) * scale + shift


@pytest.mark.parametrize("eps", [1e-5, 0.5])
def test_params_match_torch_autograd_f64(eps):
    x = _rand(7, 45, 30, scale=3.0, shift=0.5)
    dy = _rand(7, 45, 31)
    g = torch.tensor(np.random.default_rng(32).uniform(0.5, 1.5, 45), requires_grad=True)
    b = torch.tensor(np.random.default_rng(33).standard_normal(45), requires_grad=True)
    y = torch.nn.functional.layer_norm(torch.tensor(x), (45,), g, b, eps=eps)
    y.backward(torch.tensor(dy))
    dgam, dbet = oracle.layernorm_backward_params(x, dy, eps)
    np.testing.assert_allclose(dgam, g.grad.numpy(), rtol=1e-12, atol=1e-13 * np.abs(dgam).max())
    np.testing.assert_allclose(dbet, b.grad.numpy(), rtol=1e-13, atol=1e-14)


def test_params_finite_difference_of_forward_oracle():
    rng = np.random.default_rng(34)
    rows, cols = 6, 19
    x = rng.standard_normal((rows, cols)) * 2 + 1
    dy = rng.standard_normal((rows, cols))
    gamma = rng.uniform(0.5, 1.5, cols)
    beta = rng.standard_normal(cols)
    eps = 1e-3
    dgam, dbet = oracle.layernorm_backward_params(x, dy, eps)

    def loss(gm, bt):
        return float((dy * oracle.layernorm(x, gm, bt, eps)).sum())
    base = loss(gamma, beta)
    for j in range(cols):
        e = np.zeros(cols)
        e[j] = 1.0
        # linear in gamma and beta: a unit step is exact up to rounding
        assert abs((loss(gamma + e, beta) - base) - dgam[j]) <= 1e-12 * np.abs(dy).sum()
        assert abs((loss(gamma, beta + e) - base) - dbet[j]) <= 1e-12 * np.abs(dy).sum()


def test_row_stats_match_numpy():
    x = _rand(9, 101, 35, scale=4.0, shift=-2.0)
    for eps in (1e-5, 0.3):
        mu, rstd = oracle.layernorm_row_stats(x, eps)
        np.testing.assert_allclose(mu, x.mean(axis=1), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(rstd, 1.0 / np.sqrt(x.var(axis=1) + eps), rtol=1e-13)


def test_params_closed_forms():
    x = _rand(5, 12, 36, scale=2.0, shift=3.0)
    eps = 1e-5
    mu = x.mean(axis=1, keepdims=True)
    xhat = (x - mu) / np.sqrt(x.var(axis=1, keepdims=True) + eps)
    # one row: the elementwise products
    dg1, db1 = oracle.layernorm_backward_params(x[:1], x[1:2] * 2.0, eps)
    np.testing.assert_allclose(dg1, 2.0 * x[1] * xhat[0], rtol=1e-12)
    np.testing.assert_allclose(db1, 2.0 * x[1], rtol=1e-15)
    # a constant dy: dbeta = rows * c, dgamma = c * column sums of xhat
    dg, db = oracle.layernorm_backward_params(x, np.full_like(x, 0.5), eps)
    np.testing.assert_allclose(db, 2.5, rtol=1e-15)
    np.testing.assert_allclose(dg, 0.5 * xhat.sum(axis=0), rtol=1e-11, atol=1e-13)
    # and each row's xhat sums to zero, so the dgamma entries do too
    assert abs(dg.sum()) < 1e-12
    # dy = xhat: dgamma_j = sum_i xhat_ij^2, and sum_j dgamma_j = rows * cols * v / (v + eps)
    dg, _ = oracle.layernorm_backward_params(x, xhat, eps)
    np.testing.assert_allclose(dg, (xhat ** 2).sum(axis=0), rtol=1e-12)
    v = x.var(axis=1)
    np.testing.assert_allclose(dg.sum(), (12 * v / (v + eps)).sum(), rtol=1e-12)


def test_params_empty_and_degenerate():
    dg, db = oracle.layernorm_backward_params(np.zeros((0, 8)), np.zeros((0, 8)), 1e-5)
    assert dg.shape == (8,) and not dg.any() and not db.any()
    # a constant row has xhat = 0: it adds to dbeta only
    x = np.vstack([np.full(8, 3.0), _rand(1, 8, 37)[0]])
    dy = _rand(2, 8, 38)
    dg, db = oracle.layernorm_backward_params(x, dy, 1e-5)
    dg2, _ = oracle.layernorm_backward_params(x[1:], dy[1:], 1e-5)
    np.testing.assert_allclose(dg, dg2, rtol=1e-15)
    np.testing.assert_allclose(db, dy.sum(axis=0), rtol=1e-15)
