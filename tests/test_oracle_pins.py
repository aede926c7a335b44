"""Pins for the CPU oracle: closed forms, invariants, hand-derived worked examples,
brute force in 50-digit decimal arithmetic and library routines.

Each test targets a mistake the oracle could plausibly contain (a dropped term, a
wrong sign, a transposed operand, a biased/unbiased mix-up, eps in the wrong
place, a wrong merge rule).  The operator definitions are the reduction-reuse
instances of the CREDIT paper (Sec. III-B, Eq. 1); the slice/merge identity is
Eq. 2 of the same section.
"""
import decimal
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = np.array([float(v) for v in nums])
    return vals


# ---------------------------------------------------------------------------
# worked examples (hand-derived, tests/golden)
# ---------------------------------------------------------------------------
def test_golden_softmax_logs():
    g = _read_golden("softmax_logs.txt")
    y = oracle.softmax(g["x"])[0]
    np.testing.assert_allclose(y, g["y"], rtol=1e-15, atol=0)


def test_golden_layernorm_1234():
    g = _read_golden("layernorm_1234.txt")
    y = oracle.layernorm(g["x"], g["gamma"], g["beta"], float(g["eps"][0]))[0]
    np.testing.assert_allclose(y, g["y"], rtol=1e-15, atol=1e-15)


def test_golden_rmsnorm_34():
    g = _read_golden("rmsnorm_34.txt")
    y = oracle.rmsnorm(g["x"], g["gamma"], float(g["eps"][0]))[0]
    np.testing.assert_allclose(y, g["y"], rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# softmax
# ---------------------------------------------------------------------------
def _rand(rows, cols, seed, scale=1.0, shift=0.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols)) * scale + shift


def test_softmax_rows_sum_to_one_nonsquare():
    x = _rand(7, 33, 0, scale=3.0)
    y = oracle.softmax(x)
    assert y.shape == (7, 33)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=33 * 2.0 ** -52)
    assert np.all(y > 0)


@pytest.mark.parametrize("c", [-50.0, 50.0, 1000.0, -1000.0])
def test_softmax_shift_invariance(c):
    # A missing max subtraction overflows (or underflows to 0/0) at |c| = 1000.
    x = _rand(5, 40, 1)
    np.testing.assert_allclose(oracle.softmax(x + c), oracle.softmax(x), rtol=2e-12, atol=0)


def test_softmax_constant_row_is_uniform():
    for n in (1, 3, 64, 1000):
        y = oracle.softmax(np.full((2, n), -7.25))
        assert np.all(y == 1.0 / n)


def test_softmax_two_elements_is_logistic():
    rng = np.random.default_rng(2)
    for _ in range(20):
        a, b = rng.standard_normal(2) * 4
        y = oracle.softmax([[a, b]])[0]
        assert abs(y[0] - 1.0 / (1.0 + math.exp(b - a))) <= 1e-15
        assert abs(y[1] - 1.0 / (1.0 + math.exp(a - b))) <= 1e-15


def test_softmax_dominant_element_is_one_hot():
    x = np.zeros((1, 50))
    x[0, 17] = 800.0
    y = oracle.softmax(x)[0]
    assert y[17] == 1.0
    assert np.all(np.delete(y, 17) == 0.0)


def test_softmax_matches_torch_f64():
    x = _rand(9, 257, 3, scale=5.0)
    ref = torch.softmax(torch.from_numpy(x), dim=-1).numpy()
    np.testing.assert_allclose(oracle.softmax(x), ref, rtol=1e-12, atol=0)


def test_softmax_with_logits_masked_to_the_lowest_float():
    # logits masked with the lowest finite float32 (as a masked fill does):
    # those entries are exactly 0 and the rest is the softmax of the unmasked
    # entries alone (torch float64 on the subset); a fully masked row is
    # uniform, 1/N exactly
    low = float(np.finfo(np.float32).min)
    x = _rand(3, 64, 11, scale=3.0)
    mask = np.zeros_like(x, dtype=bool)
    mask[0, ::3] = True
    mask[1, 1:] = True
    mask[2, :] = True
    x[mask] = low
    y = oracle.softmax(x)
    assert np.all(y[0][mask[0]] == 0.0) and np.all(y[1][mask[1]] == 0.0)
    for r in (0, 1):
        keep = ~mask[r]
        ref = torch.softmax(torch.from_numpy(x[r][keep]), dim=-1).numpy()
        np.testing.assert_allclose(y[r][keep], ref, rtol=1e-12, atol=0)
    assert np.all(y[2] == 1.0 / 64)


def test_softmax_nan_propagates_to_row():
    x = _rand(2, 16, 4)
    x[1, 5] = np.nan
    y = oracle.softmax(x)
    assert np.all(np.isfinite(y[0])) and np.all(np.isnan(y[1]))


# ---------------------------------------------------------------------------
# LayerNorm
# ---------------------------------------------------------------------------
def test_layernorm_unit_affine_mean_zero_and_variance_closed_form():
    # With gamma = 1, beta = 0: mean(y) = 0 and biased var(y) = v / (v + eps).
    # Small-variance rows make eps visible, so eps outside the root, an
    # unbiased variance or a dropped eps all fail.
    rng = np.random.default_rng(5)
    n = 200
    eps = 1e-5
    for scale in (1e-3, 3e-3, 1.0):
        x = rng.standard_normal((4, n)) * scale + 0.5
        y = oracle.layernorm(x, np.ones(n), np.zeros(n), eps)
        v = x.var(axis=1)  # numpy's default is the biased (1/N) variance
        np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
        np.testing.assert_allclose(y.var(axis=1), v / (v + eps), rtol=1e-12)


def test_layernorm_constant_row_gives_beta():
    n = 16
    gamma = np.linspace(0.5, 1.5, n)
    beta = np.linspace(-1.0, 2.0, n)
    y = oracle.layernorm(np.full((3, n), 3.25), gamma, beta, 1e-5)
    assert np.all(y == beta)


def test_layernorm_two_elements_closed_form():
    rng = np.random.default_rng(6)
    eps = 1e-3
    for _ in range(20):
        a, b = rng.standard_normal(2)
        g = rng.uniform(0.5, 1.5, 2)
        bt = rng.standard_normal(2)
        d = (a - b) / 2
        y = oracle.layernorm([[a, b]], g, bt, eps)[0]
        r = d / math.sqrt(d * d + eps)
        np.testing.assert_allclose(y, [r * g[0] + bt[0], -r * g[1] + bt[1]], rtol=1e-13, atol=1e-15)


def test_layernorm_affine_invariance_eps0():
    x = _rand(3, 100, 7)
    g = np.ones(100)
    z = np.zeros(100)
    np.testing.assert_allclose(oracle.layernorm(2.5 * x - 11.0, g, z, 0.0),
                               oracle.layernorm(x, g, z, 0.0), rtol=1e-11, atol=1e-12)


def test_layernorm_matches_torch_f64():
    x = _rand(6, 130, 8, scale=3.0, shift=0.5)
    rng = np.random.default_rng(9)
    g = rng.uniform(0.5, 1.5, 130)
    b = rng.standard_normal(130) * 0.1
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (130,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layernorm(x, g, b, 1e-5), ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def test_rmsnorm_constant_row():
    n = 32
    g = np.linspace(0.5, 1.5, n)
    eps = 1e-6
    for c in (-3.0, 0.02, 7.5):
        y = oracle.rmsnorm(np.full((2, n), c), g, eps)
        np.testing.assert_allclose(y, np.broadcast_to(c / math.sqrt(c * c + eps) * g, (2, n)),
                                   rtol=1e-15)
        # "constant row -> gamma * sign" to within eps / (2 c^2)
        assert np.all(np.abs(y - math.copysign(1.0, c) * g) <= g * eps / (2 * c * c) * 1.01)


def test_rmsnorm_scale_invariance_eps0():
    x = _rand(3, 77, 10)
    g = np.ones(77)
    np.testing.assert_allclose(oracle.rmsnorm(4.0 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(-0.25 * x, g, 0.0), -oracle.rmsnorm(x, g, 0.0), rtol=1e-14)


def test_rmsnorm_mean_square_closed_form():
    rng = np.random.default_rng(11)
    eps = 1e-6
    x = rng.standard_normal((5, 150)) * np.array([[1e-3], [1.0], [30.0], [2e-3], [0.5]])
    y = oracle.rmsnorm(x, np.ones(150), eps)
    ms = (x * x).mean(axis=1)
    np.testing.assert_allclose((y * y).mean(axis=1), ms / (ms + eps), rtol=1e-13)


def test_rmsnorm_matches_torch_f64():
    x = _rand(5, 96, 12)
    g = np.random.default_rng(13).uniform(0.5, 1.5, 96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-6), ref, rtol=1e-13)


# ---------------------------------------------------------------------------
# 50-digit decimal brute force on tiny rows
# ---------------------------------------------------------------------------
def _dec_softmax(row):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        d = [decimal.Decimal(float(v)) for v in row]
        m = max(d)
        e = [(v - m).exp() for v in d]
        s = sum(e)
        return [float(v / s) for v in e]


def _dec_layernorm(row, g, b, eps):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        d = [decimal.Decimal(float(v)) for v in row]
        n = len(d)
        mu = sum(d) / n
        var = sum((v - mu) ** 2 for v in d) / n
        den = (var + decimal.Decimal(eps)).sqrt()
        return [float((v - mu) / den * decimal.Decimal(float(gi)) + decimal.Decimal(float(bi)))
                for v, gi, bi in zip(d, g, b)]


def _dec_rmsnorm(row, g, eps):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        d = [decimal.Decimal(float(v)) for v in row]
        ms = sum(v * v for v in d) / len(d)
        den = (ms + decimal.Decimal(eps)).sqrt()
        return [float(v / den * decimal.Decimal(float(gi))) for v, gi in zip(d, g)]


@pytest.mark.parametrize("n", [1, 2, 5, 17, 64])
def test_decimal_brute_force(n):
    rng = np.random.default_rng(100 + n)
    x = rng.standard_normal((3, n)) * 3 + 0.5
    g = rng.uniform(0.5, 1.5, n)
    b = rng.standard_normal(n) * 0.1
    eps = float(np.float32(1e-5))
    ys = oracle.softmax(x)
    yl = oracle.layernorm(x, g, b, eps)
    yr = oracle.rmsnorm(x, g, eps)
    for r in range(3):
        np.testing.assert_allclose(ys[r], _dec_softmax(x[r]), rtol=1e-14, atol=0)
        np.testing.assert_allclose(yl[r], _dec_layernorm(x[r], g, b, eps), rtol=0, atol=1e-13)
        np.testing.assert_allclose(yr[r], _dec_rmsnorm(x[r], g, eps), rtol=1e-14, atol=0)


# ---------------------------------------------------------------------------
# Eq. 2: slice partials and their combination are partition invariant
# ---------------------------------------------------------------------------
def _random_bounds(rng, n, p, allow_empty=True):
    cuts = np.sort(rng.integers(0 if allow_empty else 1, n + (1 if allow_empty else 0), size=p - 1))
    return np.concatenate([[0], cuts, [n]]).astype(np.int64)


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_softmax_merge_partition_invariance(p):
    rng = np.random.default_rng(20 + p)
    for trial in range(20):
        n = int(rng.integers(p, 300))
        x = rng.standard_normal(n) * 4 + rng.uniform(-50, 50)
        m_ref, s_ref = oracle.softmax_stats(x)
        b = _random_bounds(rng, n, p)
        m_c, s_c = oracle.softmax_partials(x, b)
        m, s = oracle.softmax_merge(m_c, s_c)
        assert m == m_ref[0]
        assert abs(s - s_ref[0]) <= 1e-12 * s_ref[0]


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_layernorm_merge_partition_invariance(p):
    rng = np.random.default_rng(40 + p)
    for trial in range(20):
        n = int(rng.integers(p, 300))
        x = rng.standard_normal(n) * 3 + 0.5
        mu_ref, m2_ref = oracle.layernorm_stats(x)
        b = _random_bounds(rng, n, p)
        n_c, mu_c, m2_c = oracle.layernorm_partials(x, b)
        nn, mu, m2 = oracle.layernorm_merge(n_c, mu_c, m2_c)
        assert nn == n
        assert abs(mu - mu_ref[0]) <= 1e-12 * max(1.0, abs(mu_ref[0]))
        assert abs(m2 - m2_ref[0]) <= 1e-12 * m2_ref[0]


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_rmsnorm_partials_sum_to_full(p):
    rng = np.random.default_rng(60 + p)
    for trial in range(20):
        n = int(rng.integers(p, 300))
        x = rng.standard_normal(n)
        b = _random_bounds(rng, n, p)
        ss = oracle.rmsnorm_partials(x, b)
        assert abs(ss.sum() - float(np.dot(x, x))) <= 1e-12 * float(np.dot(x, x))
        # each slice partial is its own sum of squares (catches an index slip)
        for c in range(p):
            seg = x[b[c]:b[c + 1]]
            assert abs(ss[c] - float(np.dot(seg, seg))) <= 1e-13 * max(1.0, float(np.dot(seg, seg)))


def test_merge_identity_elements_and_associativity():
    rng = np.random.default_rng(70)
    x = rng.standard_normal(64) * 2
    # an empty slice is the identity
    m_c, s_c = oracle.softmax_partials(x, [0, 0, 64])
    assert m_c[0] == -np.inf and s_c[0] == 0.0
    n_c, mu_c, m2_c = oracle.layernorm_partials(x, [0, 64, 64])
    assert n_c[1] == 0 and m2_c[1] == 0.0
    # associativity: merging (a (b c)) and ((a b) c) agree
    b = [0, 10, 40, 64]
    m_c, s_c = oracle.softmax_partials(x, b)
    m_ab, s_ab = oracle.softmax_merge(m_c[:2], s_c[:2])
    m_bc, s_bc = oracle.softmax_merge(m_c[1:], s_c[1:])
    left = oracle.softmax_merge([m_ab, m_c[2]], [s_ab, s_c[2]])
    right = oracle.softmax_merge([m_c[0], m_bc], [s_c[0], s_bc])
    assert left[0] == right[0] and abs(left[1] - right[1]) <= 1e-13 * left[1]
    n_c, mu_c, m2_c = oracle.layernorm_partials(x, b)
    ab = oracle.layernorm_merge(n_c[:2], mu_c[:2], m2_c[:2])
    bc = oracle.layernorm_merge(n_c[1:], mu_c[1:], m2_c[1:])
    left = oracle.layernorm_merge([ab[0], n_c[2]], [ab[1], mu_c[2]], [ab[2], m2_c[2]])
    right = oracle.layernorm_merge([n_c[0], bc[0]], [mu_c[0], bc[1]], [m2_c[0], bc[2]])
    np.testing.assert_allclose(left, right, rtol=1e-13)


# ---------------------------------------------------------------------------
# double -> bf16 rounding (nearest, ties to even, directly from double)
# ---------------------------------------------------------------------------
def _bits(v):
    return int(oracle.round_bf16(np.array([v]))[0])


def test_bf16_rounding_matches_torch_on_float_patterns():
    # Every float32 exponent and sign, with low halves that exercise ties,
    # just-below/above-tie, zero and all-ones, plus random low halves.
    rng = np.random.default_rng(80)
    hi = np.arange(65536, dtype=np.uint32)
    lows = np.concatenate([[0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF],
                           rng.integers(0, 65536, 26)]).astype(np.uint32)
    pats = ((hi[:, None] << np.uint32(16)) | lows[None, :]).reshape(-1)
    f = pats.view(np.float32)
    finite = np.isfinite(f)
    f = f[finite]
    got = oracle.round_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_special_cases():
    one = 0x3F80
    assert _bits(1.0 + 2.0 ** -8) == one                     # tie -> even (down)
    assert _bits(1.0 + 3 * 2.0 ** -8) == one + 2             # tie -> even (up)
    # direct rounding from double: just above the tie rounds up, whereas going
    # through float first would land exactly on the tie and round down
    assert _bits(1.0 + 2.0 ** -8 + 2.0 ** -40) == one + 1
    assert _bits(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0x8000 | (one + 1)
    bf16_max = 255.0 * 2.0 ** 120
    half_ulp = 2.0 ** 119
    assert _bits(bf16_max) == 0x7F7F
    assert _bits(bf16_max + half_ulp * 0.99) == 0x7F7F
    assert _bits(bf16_max + half_ulp) == 0x7F80                # tie above max -> inf
    assert _bits(2.0 ** -134) == 0x0000                         # half of min subnormal -> 0 (even)
    assert _bits(3 * 2.0 ** -134) == 0x0002                     # 1.5 * min subnormal -> 2 * min
    assert _bits(2.0 ** -133) == 0x0001
    assert _bits(-0.0) == 0x8000
    assert _bits(float("inf")) == 0x7F80
    assert _bits(float("nan")) & 0x7FC0 == 0x7FC0
