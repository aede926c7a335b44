"""Pins for the oracle of the three further reduction-reuse workloads of the
CREDIT paper's evaluation (Sec. IV-A; traffic in Sec. IV-D and Fig. 5):
softmax-logits backward, LayerNorm backward (row part) and row-wise int8
quantization.

The backward oracles are pinned to torch's float64 autograd (a library
routine), to central finite differences of the already pinned forward oracles
(an independent route to the same derivative), and to closed forms and
invariants.  The quantizer is pinned to hand-derived worked examples
(tests/golden) and to properties any correct quantizer has: the bound on the
dequantization error, symmetry, exact power-of-two scaling, monotonicity.
The slice/merge identities (Eq. 2) of the two backward partials are checked
against the plain per-row statistics for random partitions.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rows, cols, seed, scale=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols)) * scale + shift


# ---------------------------------------------------------------------------
# softmax-logits backward
# ---------------------------------------------------------------------------
def _torch_softmax_grad(x, dy):
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    torch.softmax(xt, dim=-1).backward(torch.tensor(dy, dtype=torch.float64))
    return xt.grad.numpy()


def test_softmax_backward_matches_torch_autograd_f64():
    x = _rand(6, 77, 1, scale=4.0, shift=3.0)
    dy = _rand(6, 77, 2)
    ref = _torch_softmax_grad(x, dy)
    got = oracle.softmax_backward(x, dy)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())


def test_softmax_backward_finite_difference_of_forward_oracle():
    # d/dt sum_i dy_i softmax(x + t v)_i at t = 0 equals sum_i dx_i v_i
    rng = np.random.default_rng(3)
    x = rng.standard_normal(40) * 2
    dy = rng.standard_normal(40)
    dx = oracle.softmax_backward(x, dy)[0]
    for _ in range(5):
        v = rng.standard_normal(40)
        h = 1e-4
        lp = float(dy @ oracle.softmax(x + h * v)[0])
        lm = float(dy @ oracle.softmax(x - h * v)[0])
        fd = (lp - lm) / (2 * h)
        assert abs(fd - float(dx @ v)) <= 1e-7 * float(np.abs(dx) @ np.abs(v))


def test_softmax_backward_rows_sum_to_zero():
    x = _rand(5, 300, 4, scale=3.0)
    dy = _rand(5, 300, 5)
    dx = oracle.softmax_backward(x, dy)
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=300 * 2.0 ** -52 * np.abs(dy).max())


@pytest.mark.parametrize("c", [-1000.0, 50.0])
def test_softmax_backward_shift_invariances(c):
    # shifting the logits changes nothing (a missing max subtraction overflows
    # at |c| = 1000); shifting dy by a constant changes nothing either (the
    # dot product term removes it)
    x = _rand(4, 50, 6)
    dy = _rand(4, 50, 7)
    ref = oracle.softmax_backward(x, dy)
    np.testing.assert_allclose(oracle.softmax_backward(x + c, dy), ref, rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(oracle.softmax_backward(x, dy + c / 100), ref, rtol=1e-9,
                               atol=1e-12 * np.abs(ref).max())


def test_softmax_backward_two_elements_closed_form():
    # p0 = sigma(a - b): dx0 = p0 p1 (dy0 - dy1) = -dx1
    for a, b, g0, g1 in [(0.3, -1.2, 2.0, -0.5), (5.0, 5.0, 1.0, 0.0), (-3.0, 4.0, 0.25, 7.0)]:
        p0 = 1.0 / (1.0 + np.exp(-(a - b)))
        p1 = 1.0 - p0
        dx = oracle.softmax_backward([a, b], [g0, g1])[0]
        np.testing.assert_allclose(dx, [p0 * p1 * (g0 - g1), -p0 * p1 * (g0 - g1)], rtol=1e-13)


def test_softmax_backward_unit_dy_is_jacobian_column():
    # dy = e_k gives column k of the softmax Jacobian: dx_i = p_k (delta_ik - p_i)
    x = _rand(1, 9, 8)[0]
    p = oracle.softmax(x)[0]
    for k in (0, 4, 8):
        dy = np.zeros(9)
        dy[k] = 1.0
        expect = -p * p[k]
        expect[k] += p[k]
        np.testing.assert_allclose(oracle.softmax_backward(x, dy)[0], expect, rtol=1e-13, atol=1e-17)


# ---------------------------------------------------------------------------
# LayerNorm backward (row part)
# ---------------------------------------------------------------------------
def _torch_layernorm_grad(x, dy, gamma, eps):
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    g = torch.tensor(gamma, dtype=torch.float64)
    beta = torch.full_like(g, 0.3)
    y = torch.nn.functional.layer_norm(xt, (x.shape[1],), g, beta, eps=eps)
    y.backward(torch.tensor(dy, dtype=torch.float64))
    return xt.grad.numpy()


@pytest.mark.parametrize("eps", [1e-5, 0.5])
def test_layernorm_backward_matches_torch_autograd_f64(eps):
    x = _rand(5, 61, 10, scale=3.0, shift=0.5)
    dy = _rand(5, 61, 11)
    gamma = np.random.default_rng(12).uniform(0.5, 1.5, 61)
    ref = _torch_layernorm_grad(x, dy, gamma, eps)
    got = oracle.layernorm_backward(x, dy, gamma, eps)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())


def test_layernorm_backward_finite_difference_of_forward_oracle():
    rng = np.random.default_rng(13)
    n = 33
    x = rng.standard_normal(n) * 2 + 1
    dy = rng.standard_normal(n)
    gamma = rng.uniform(0.5, 1.5, n)
    beta = rng.standard_normal(n)
    eps = 1e-3
    dx = oracle.layernorm_backward(x, dy, gamma, eps)[0]
    for _ in range(5):
        v = rng.standard_normal(n)
        h = 1e-4
        lp = float(dy @ oracle.layernorm(x + h * v, gamma, beta, eps)[0])
        lm = float(dy @ oracle.layernorm(x - h * v, gamma, beta, eps)[0])
        fd = (lp - lm) / (2 * h)
        assert abs(fd - float(dx @ v)) <= 1e-7 * float(np.abs(dx) @ np.abs(v))


def test_layernorm_backward_invariants():
    x = _rand(4, 128, 14, scale=3.0, shift=0.5)
    dy = _rand(4, 128, 15)
    gamma = np.random.default_rng(16).uniform(0.5, 1.5, 128)
    dx = oracle.layernorm_backward(x, dy, gamma, 1e-5)
    scale = np.abs(dx).max()
    # the gradient is orthogonal to the all-ones direction ...
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-12 * 128 * scale)
    # ... and, at eps = 0, to x itself (LayerNorm ignores scaling of x)
    dx0 = oracle.layernorm_backward(x, dy, gamma, 0.0)
    np.testing.assert_allclose((dx0 * x).sum(axis=1), 0.0, atol=1e-11 * 128 * np.abs(dx0).max() * np.abs(x).max())
    # shift invariance, and 1/alpha scaling at eps = 0
    np.testing.assert_allclose(oracle.layernorm_backward(x + 7.0, dy, gamma, 1e-5), dx, rtol=1e-9,
                               atol=1e-12 * scale)
    np.testing.assert_allclose(oracle.layernorm_backward(x * 4.0, dy, gamma, 0.0), dx0 / 4.0, rtol=1e-10,
                               atol=1e-13 * np.abs(dx0).max())


def test_layernorm_backward_constant_g_gives_zero():
    # gamma * dy constant: the mean removes it and it is orthogonal to xhat
    x = _rand(1, 20, 17)[0]
    gamma = np.random.default_rng(18).uniform(0.5, 1.5, 20)
    dx = oracle.layernorm_backward(x, 0.75 / gamma, gamma, 1e-5)[0]
    np.testing.assert_allclose(dx, 0.0, atol=1e-14)


def test_layernorm_backward_g_equal_xhat_closed_form():
    # g = xhat: dx_i = rstd (xhat_i - xhat_i mean(xhat^2)) = rstd xhat_i eps / (v + eps)
    x = _rand(1, 24, 19, scale=2.0)[0]
    eps = 0.25
    mu = x.mean()
    v = ((x - mu) ** 2).mean()
    rstd = 1.0 / np.sqrt(v + eps)
    xhat = (x - mu) * rstd
    gamma = np.random.default_rng(20).uniform(0.5, 1.5, 24)
    dx = oracle.layernorm_backward(x, xhat / gamma, gamma, eps)[0]
    np.testing.assert_allclose(dx, rstd * xhat * eps / (v + eps), rtol=1e-12, atol=1e-15)


def test_layernorm_backward_two_elements_closed_form():
    # x = (a, b), d = (a - b) / 2: dx0 = -dx1 = rstd (g0 - g1) / 2 * eps / (d^2 + eps)
    for a, b, g0, g1, eps in [(1.0, -2.0, 0.5, 3.0, 0.1), (4.0, 4.5, -1.0, 2.0, 1e-5)]:
        d = (a - b) / 2
        rstd = 1.0 / np.sqrt(d * d + eps)
        want = rstd * (g0 - g1) / 2 * eps / (d * d + eps)
        dx = oracle.layernorm_backward([a, b], [g0, g1], [1.0, 1.0], eps)[0]
        np.testing.assert_allclose(dx, [want, -want], rtol=1e-12)


# ---------------------------------------------------------------------------
# Eq. 2 for the backward partials
# ---------------------------------------------------------------------------
def _random_bounds(rng, n, p):
    cuts = np.sort(rng.integers(0, n + 1, size=p - 1))
    return np.concatenate([[0], cuts, [n]]).astype(np.int64)


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_softmax_backward_merge_partition_invariance(p):
    rng = np.random.default_rng(30 + p)
    for _ in range(20):
        n = int(rng.integers(p, 300))
        x = rng.standard_normal(n) * 4 + rng.uniform(-50, 50)
        dy = rng.standard_normal(n)
        m_ref, s_ref, u_ref = oracle.softmax_backward_stats(x, dy)
        b = _random_bounds(rng, n, p)
        m, s, u = oracle.softmax_backward_merge(*oracle.softmax_backward_partials(x, dy, b))
        assert m == m_ref[0]
        assert abs(s - s_ref[0]) <= 1e-12 * s_ref[0]
        assert abs(u - u_ref[0]) <= 1e-12 * float(np.abs(dy).max()) * s_ref[0]
    # each slice partial is its own slice's sums (catches an index slip)
    x = rng.standard_normal(50)
    dy = rng.standard_normal(50)
    m_c, s_c, u_c = oracle.softmax_backward_partials(x, dy, [0, 20, 50])
    m2, s2, u2 = oracle.softmax_backward_stats(x[20:], dy[20:])
    assert (m_c[1], s_c[1]) == (m2[0], s2[0]) and abs(u_c[1] - u2[0]) <= 1e-13 * s2[0]


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_layernorm_backward_merge_partition_invariance(p):
    rng = np.random.default_rng(50 + p)
    for _ in range(20):
        n = int(rng.integers(p, 300))
        x = rng.standard_normal(n) * 3 + rng.uniform(-20, 20)
        g = rng.standard_normal(n)
        mu_ref, m2_ref, a_ref, b_ref = oracle.layernorm_backward_stats(x, g)
        b = _random_bounds(rng, n, p)
        nn, mu, m2, a, bb = oracle.layernorm_backward_merge(*oracle.layernorm_backward_partials(x, g, b))
        assert nn == n
        scale = float(np.abs(g) @ np.abs(x - mu_ref[0]))
        assert abs(mu - mu_ref[0]) <= 1e-12 * max(1.0, abs(mu_ref[0]))
        assert abs(m2 - m2_ref[0]) <= 1e-11 * m2_ref[0]
        assert abs(a - a_ref[0]) <= 1e-12 * float(np.abs(g).sum())
        assert abs(bb - b_ref[0]) <= 1e-11 * scale


def test_backward_merge_identity_elements():
    x = np.arange(10.0)
    g = np.ones(10)
    m_c, s_c, u_c = oracle.softmax_backward_partials(x, g, [0, 0, 10])
    assert m_c[0] == -np.inf and s_c[0] == 0.0 and u_c[0] == 0.0
    n_c, mu_c, m2_c, a_c, b_c = oracle.layernorm_backward_partials(x, g, [0, 10, 10])
    assert n_c[1] == 0 and a_c[1] == 0 and b_c[1] == 0


# ---------------------------------------------------------------------------
# int8 quantization
# ---------------------------------------------------------------------------
def _nearest_f32(num, den):
    """The float32 nearest to num / den (exact rational arithmetic)."""
    q = Fraction(int(num), int(den))
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    return min(cands, key=lambda c: abs(Fraction(float(c)) - q))


def _golden_rows():
    rows = {}
    with open(os.path.join(GOLDEN, "quantize_int8_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            rows.setdefault(key[-1], {})[key[:-1]] = [float(v) for v in nums]
    return rows


def test_golden_quantize_worked_examples():
    for name, r in sorted(_golden_rows().items()):
        q, scale = oracle.quantize_int8(np.array(r["x"], dtype=np.float32))
        assert q[0].tolist() == [int(v) for v in r["q"]], name
        assert scale[0] == _nearest_f32(*r["scale"]), name


def _quant_input(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    mask = rng.random((rows, cols)) < 0.01
    x[mask] *= 50
    return x


def test_quantize_error_bound_and_extremes():
    x = _quant_input(16, 999, 60)
    q, scale = oracle.quantize_int8(x)
    a = np.abs(x).max(axis=1)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.array_equal(scale, (a / np.float32(127)).astype(np.float32))
    # the largest element of each row maps to +-127
    arg = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(16), arg].astype(np.int32)) == 127)
    # every code is within half a step of the exact real ratio x * 127 / a
    # (plus the float roundings of inv and of the product)
    exact = x.astype(np.float64) * 127.0 / a.astype(np.float64)[:, None]
    assert np.all(np.abs(q - exact) <= 0.5 + 2e-5)
    # and dequantizes to within half a step
    assert np.all(np.abs(q * scale[:, None].astype(np.float64) - x) <= scale[:, None] * (0.5 + 2e-5))


def test_quantize_symmetry_scaling_monotonicity():
    x = _quant_input(8, 257, 61)
    q, s = oracle.quantize_int8(x)
    qn, sn = oracle.quantize_int8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # power-of-two scaling is exact in float, so the codes do not change
    q4, s4 = oracle.quantize_int8(x * np.float32(4))
    assert np.array_equal(q4, q) and np.array_equal(s4, s * np.float32(4))
    # order is preserved within a row
    for r in range(8):
        o = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(q[r][o].astype(np.int32)) >= 0)


def test_quantize_zero_and_tiny_rows():
    x = np.array([[0.0, 0.0, -0.0, 0.0], [1e-37, -5e-38, 0.0, 2e-37]], dtype=np.float32)
    q, s = oracle.quantize_int8(x)
    assert q[0].tolist() == [0, 0, 0, 0] and s[0] == 0.0
    # absmax 2e-37: 127 / a overflows and is capped at FLT_MAX, so zeros stay 0
    fmax = np.finfo(np.float32).max
    want = [int(np.rint(np.float32(v) * fmax)) for v in x[1]]
    assert want == [34, -17, 0, 68]
    assert q[1].tolist() == want


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = oracle.bf16_bits_to_f32(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
