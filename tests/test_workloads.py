"""The seeded input generators: determinism, shapes, distributions and the
float32 -> bf16 storage rounding (checked against torch's CPU conversion)."""
import numpy as np
import torch

from wide_reduction_reuse_amd import workloads as W


def test_named_configs_shapes_and_bytes():
    assert W.NAMED["softmax_f32_64x4096"].algorithmic_bytes() == 64 * 4096 * 8
    assert W.NAMED["layernorm_bf16_4096x8192"].algorithmic_bytes() == 134_250_496
    assert W.NAMED["rmsnorm_bf16_1024x65536"].algorithmic_bytes() == 268_566_528
    assert W.NAMED["softmax_f32_256x262144"].algorithmic_bytes() == 536_870_912


def test_sweep_has_90_points_with_exact_sizes():
    pts = W.sweep_points()
    assert len(pts) == 90
    assert len({p.seed for p in pts}) == 90
    for p in pts:
        assert p.rows * p.cols * p.elem_bytes in W.SWEEP_BYTES
    # spot checks of the row-count table
    by = {(p.op, p.dtype, p.cols, p.rows * p.cols * p.elem_bytes): p.rows for p in pts}
    assert by[("softmax", "f32", 1024, 16 << 20)] == 4096
    assert by[("rmsnorm", "bf16", 262144, 1 << 30)] == 2048
    assert by[("layernorm", "f32", 65536, 256 << 20)] == 1024


def test_bf16_storage_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(1 << 16) * np.exp(rng.uniform(-30, 30, 1 << 16))).astype(np.float32)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32)
    a = np.concatenate([a, ties])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(a), ref)
    back = W.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_distributed_as_stated():
    w = W.custom("layernorm", "f32", 64, 4096, seed=7, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    a = W.generate(w)
    b = W.generate(w)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.gamma, b.gamma)
    assert abs(a.x.mean() - 0.5) < 0.05 and abs(a.x.std() - 3.0) < 0.05
    assert a.gamma.min() >= 0.5 and a.gamma.max() <= 1.5
    assert abs(a.beta.std() - 0.1) < 0.01
    assert a.eps == float(np.float32(1e-5))  # default LayerNorm eps, as the float the GPU receives


def test_outliers_and_row_offsets():
    w = W.custom("rmsnorm", "f32", 64, 8192, seed=3, x_dist="outliers", outlier_prob=0.01,
                 outlier_scale=50.0)
    x = W.generate(w).x
    frac = np.mean(np.abs(x) > 8.0)
    assert 0.005 < frac < 0.012
    w = W.custom("softmax", "f32", 64, 4096, seed=4, x_dist="row_offset", x_scale=4.0, row_offset=50.0)
    x = W.generate(w).x
    means = x.mean(axis=1)
    assert means.min() < -20 and means.max() > 20 and np.abs(means).max() <= 51
    assert abs((x - means[:, None]).std() - 4.0) < 0.1


def test_scored_widths_are_never_calibrated():
    # the selector is scored on shapes the calibration never timed: the sweep
    # and off-grid widths at their sizes, the further workloads' grid rows
    calib = (W.calibration_points() + W.calibration_points_mid() + W.calibration_points_odd() +
             W.calibration_points_part())
    calib_next = W.calibration_points_next() + W.calibration_points_next_more()
    timed = {(p.op, p.dtype, p.rows, p.cols) for p in calib + calib_next}
    for p in W.sweep_points() + W.next_points() + W.offgrid_points() + W.offgrid_points_next():
        assert (p.op, p.dtype, p.rows, p.cols) not in timed, p.name
    calib_cols = {p.cols for p in calib + calib_next}
    assert not calib_cols & set(W.OFFGRID_COLS)


def test_offgrid_widths_cover_aligned_and_odd_rows():
    aligned = [c for c in W.OFFGRID_COLS if (c * 2) % 16 == 0]
    odd = [c for c in W.OFFGRID_COLS if (c * 4) % 16 != 0]
    assert len(aligned) >= 6 and len(odd) >= 3
    assert all(c % 2 == 1 for c in W.CALIB_ODD_COLS + W.CALIB_ODD_MID_COLS)
    # bf16 rows ending in a partial 16-byte vector: even, not whole vectors
    assert any((c * 2) % 16 != 0 and c % 2 == 0 for c in W.OFFGRID_COLS)
    assert all((c * 2) % 16 != 0 and c % 2 == 0 for c in W.CALIB_PART_COLS)
    assert len(set(W.CALIB_PART_COLS)) == 12
    assert all(c % 256 == 0 for c in W.CALIB_MID_COLS)
