"""The parity comparator itself (tests/parity.py), on hand-made arrays: the
rule e_i = |y_i - yhat_i| / max(|yhat_i|, tau_i) <= 1e-5 for fp32, and the
bf16 rule (2e-2 absolute after rounding the reference, or a one-ulp flip)."""
import numpy as np

from parity import FP32_TOL, compare


def test_exact_match_with_zero_scale_is_no_error():
    # a backward operator's tau is 0 where the probability underflows to 0;
    # an exact (signed) zero there must pass, any other value must not
    yhat = np.array([0.0, 0.5, -0.25])
    tau = np.array([0.0, 1.0, 1.0])
    v = compare("softmax_bwd", "f32", np.array([-0.0, 0.5, -0.25], np.float32), yhat, tau)
    assert v.ok and v.max_err == 0.0
    v = compare("softmax_bwd", "f32", np.array([1e-30, 0.5, -0.25], np.float32), yhat, tau)
    assert not v.ok and v.worst_index == 0


def test_fp32_relative_rule_and_floor():
    yhat = np.array([1.0, 1e-3])
    ok = np.array([1.0 + 0.5 * FP32_TOL, 1e-3 * (1 + 0.5 * FP32_TOL)], np.float32)
    assert compare("softmax", "f32", ok, yhat).ok
    bad = np.array([1.0, 1e-3 * (1 + 4 * FP32_TOL)], np.float32)
    assert not compare("softmax", "f32", bad, yhat).ok
    # LayerNorm's floor tau = 1: an absolute 0.5e-5 error on a near-zero output passes
    assert compare("layernorm", "f32", np.array([0.5 * FP32_TOL], np.float32), np.array([0.0])).ok


def test_nan_must_match_nan():
    yhat = np.array([np.nan, 1.0])
    assert compare("softmax", "f32", np.array([np.nan, 1.0], np.float32), yhat).ok
    assert not compare("softmax", "f32", np.array([0.0, 1.0], np.float32), yhat).ok
    assert not compare("softmax", "f32", np.array([np.nan, np.nan], np.float32), np.array([1.0, 1.0])).ok


def test_bf16_adjacent_flip_passes_two_ulps_do_not():
    # 8.0 and its bf16 neighbours: 8.0625 (one ulp up), 8.125 (two ulps)
    yhat = np.array([8.03])  # rounds to 8.0 in bf16
    one_ulp = np.array([0x4101], np.uint16)   # 8.0625
    two_ulps = np.array([0x4102], np.uint16)  # 8.125
    v = compare("layernorm", "bf16", one_ulp, yhat)
    assert v.ok and v.flips == 1
    assert not compare("layernorm", "bf16", two_ulps, yhat).ok
