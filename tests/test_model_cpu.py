"""The selector's analytic cost model (CREDIT paper, Sec. III-D, Eq. 7-9),
pinned term by term on the CPU through credit_model_terms.

The pins come from the equations' own structure, not from the constants:
Eq. 8's wave count against a brute-force count of cluster rounds, Eq. 7's
saving as the reread's share of the baseline's bytes (checked against the
bytes each operator's kernels read and write), the exchange cost growing with
P - 1 rather than P (P - 1), the idle-CU term vanishing once the baseline
fills every CU, and a negative control: a baseline that rereads nothing and
already fills the chip has nothing to gain from splitting, so the model never
picks the split there.
"""
import math
import os

import pytest

from wide_reduction_reuse_amd import credit as C


@pytest.fixture(autouse=True)
def analytic_model_only():
    C.credit_load_calibration(None)
    yield
    C.credit_load_calibration(C.CALIB_PATH if os.path.exists(C.CALIB_PATH) else None)


# bytes per element of the row inputs (what a reread reads again) and of the
# output, per operator and dtype: x (and dy for the backward operators) in,
# the row (int8 codes for quantization) out
def _io_bytes(op, dt):
    e = 4 if dt == "f32" else 2
    b_in = 2 * e if op in ("softmax_bwd", "layernorm_bwd") else e
    b_out = 1 if op == "quantize_int8" else e
    return b_in, b_out


def _rounds(rows, resident, p):
    # brute force of Eq. 8: clusters of p workgroups, as many as the device
    # holds at once (at least one, at most one per row), take rows in rounds
    clusters = max(1, min(resident // p, rows))
    done, w = 0, 0
    while done < rows:
        done += clusters
        w += 1
    return w


# rows no single workgroup holds (a path-3 baseline); every P legal but for
# LayerNorm, whose three statistics leave no room for a half row
WIDE = [("softmax", "f32", 131072), ("softmax", "bf16", 262144), ("rmsnorm", "f32", 131072),
        ("layernorm", "bf16", 262144), ("quantize_int8", "f32", 131072), ("softmax_bwd", "f32", 65536),
        ("layernorm_bwd", "f32", 65536)]


def _terms(op, dt, rows, cols, p):
    try:
        return C.credit_model_terms(op, dt, rows, cols, p)
    except C.CreditError as e:
        assert e.status == 4 and op == "layernorm" and p == 2, (op, dt, cols, p, e.status)
        return None


@pytest.mark.parametrize("op,dt,cols", WIDE)
@pytest.mark.parametrize("p", [2, 4, 8])
def test_waves_follow_eq8(op, dt, cols, p):
    for rows in (1, 7, 63, 64, 65, 255, 256, 1000, 4096, 65537):
        t = _terms(op, dt, rows, cols, p)
        if t is None:
            return
        s = t.split_resident
        assert s >= p
        assert t.waves == _rounds(rows, s, p)
        assert t.waves == math.ceil(rows / max(1, min(s // p, rows)))


@pytest.mark.parametrize("op,dt,cols", WIDE)
def test_saving_is_the_reread_share_of_the_baseline(op, dt, cols):
    b_in, b_out = _io_bytes(op, dt)
    for rows in (16, 256, 4096):
        t = C.credit_model_terms(op, dt, rows, cols, 8)
        assert t.baseline_path == 3  # no single workgroup holds these rows
        assert t.b_reread == b_in and t.b_base == 2 * b_in + b_out
        assert t.t_save_us == pytest.approx(t.t_base_us * b_in / (2 * b_in + b_out), rel=1e-12)
        # the split moves each element once: its time is at most the
        # one-read share of the baseline plus its own control and exchange
        assert t.t_split_us == pytest.approx(t.t_base_us - t.delta_us, rel=1e-12)
        assert t.delta_us == pytest.approx(t.t_save_us + t.t_occ_us - t.t_ctrl_us - t.t_dsm_us, rel=1e-9, abs=1e-9)


@pytest.mark.parametrize("op,dt,cols", WIDE)
def test_exchange_cost_grows_with_p_minus_one_not_p_times_that(op, dt, cols):
    rows = 4  # one row wave for every P
    d = {}
    for p in (2, 4, 8):
        t = _terms(op, dt, rows, cols, p)
        if t is not None:
            assert t.waves == 1
            d[p] = t.t_dsm_us
    p0 = min(d)
    assert d[p0] > 0 and len(d) >= 2
    for p in d:
        # P - 1 peers read each word; P (P - 1) would give 6 and 28 for 4 and 8 against 2
        assert d[p] / d[p0] == pytest.approx((p - 1) / (p0 - 1), rel=1e-12)
    # and it is linear in the waves: twice the rows of a full wave, twice the cost
    s = C.credit_model_terms(op, dt, 1, cols, 4).split_resident
    full = s // 4
    t1 = C.credit_model_terms(op, dt, full, cols, 4)
    t2 = C.credit_model_terms(op, dt, 2 * full, cols, 4)
    assert (t1.waves, t2.waves) == (1, 2)
    assert t2.t_dsm_us == pytest.approx(2 * t1.t_dsm_us, rel=1e-12)


def test_exchange_words_scale_with_the_statistics_per_partial():
    # q: softmax exchanges (max, sum), RMSNorm one sum of squares, LayerNorm
    # (count, mean, M2), quantization one absolute maximum
    q = {}
    for op in ("softmax", "rmsnorm", "layernorm", "quantize_int8"):
        q[op] = C.credit_model_terms(op, "f32", 4, 131072, 4).t_dsm_us
    assert q["softmax"] / q["rmsnorm"] == pytest.approx(2.0, rel=1e-12)
    assert q["layernorm"] / q["rmsnorm"] == pytest.approx(3.0, rel=1e-12)
    assert q["quantize_int8"] == pytest.approx(q["rmsnorm"], rel=1e-12)


@pytest.mark.parametrize("op,dt,cols", WIDE)
def test_idle_cu_term(op, dt, cols):
    for p in (2, 4, 8):
        for rows in (1, 16, 100, 255, 256, 257, 4096):
            t = _terms(op, dt, rows, cols, p)
            if t is None:
                break
            u_base = min(1.0, rows / 256)
            u_split = min(1.0, rows * p / 256)
            assert t.t_occ_us == pytest.approx((t.t_base_us - t.t_save_us) * (1 - u_base / u_split),
                                               rel=1e-9, abs=1e-12)
            if rows >= 256:
                assert t.t_occ_us == 0.0


NO_REREAD = [("layernorm", "bf16", 4096, 8192), ("softmax", "f32", 8192, 4096), ("rmsnorm", "bf16", 2048, 16384),
             ("softmax", "bf16", 16384, 2048), ("quantize_int8", "f32", 4096, 8192),
             ("layernorm_bwd", "f32", 4096, 4096)]


@pytest.mark.parametrize("op,dt,rows,cols", NO_REREAD)
def test_negative_control_no_reread_and_a_full_chip_never_splits(op, dt, rows, cols):
    # a row one workgroup holds is read once (b_reread = 0), and rows >= 256
    # owners leave no CU idle: nothing is saved, so dT < 0 for every P and the
    # selector keeps path 1
    any_legal = False
    for p in (2, 4, 8):
        try:
            t = C.credit_model_terms(op, dt, rows, cols, p)
        except C.CreditError as e:
            assert e.status == 4
            continue
        any_legal = True
        assert t.baseline_path == 1
        assert t.b_reread == 0 and t.t_save_us == 0 and t.t_occ_us == 0
        assert t.delta_us < 0 and t.t_split_us > t.t_base_us
    assert any_legal
    assert C.credit_select_path(op, dt, rows, cols).path == 1


@pytest.mark.parametrize("op,dt,rows,cols", [("softmax", "f32", 256, 262144), ("softmax", "f32", 16, 262144),
                                              ("rmsnorm", "bf16", 64, 65536), ("layernorm", "f32", 1024, 65536),
                                              ("softmax", "bf16", 4096, 8192), ("quantize_int8", "bf16", 33, 100003)])
def test_selector_splits_exactly_when_some_p_gains(op, dt, rows, cols):
    deltas = {}
    for p in (2, 4, 8):
        try:
            deltas[p] = C.credit_model_terms(op, dt, rows, cols, p)
        except C.CreditError:
            pass
    plan = C.credit_select_path(op, dt, rows, cols)
    if not deltas:
        assert plan.path != 2
        return
    best = min(deltas, key=lambda p: deltas[p].t_split_us)
    if deltas[best].delta_us > 0:
        assert plan.path == 2 and plan.split_p == best
        assert plan.predicted_us[1] == pytest.approx(deltas[best].t_split_us, rel=1e-12)
    else:
        assert plan.path == deltas[best].baseline_path


def test_model_terms_reject_bad_arguments():
    for args in [("softmax", "f32", 0, 1024, 2), ("softmax", "f32", 4, 0, 2), ("softmax", "f32", 4, 1024, 3),
                 ("softmax", "f32", 4, 1024, 16)]:
        with pytest.raises(C.CreditError) as e:
            C.credit_model_terms(*args)
        assert e.value.status == 1
    assert C.lib().credit_model_terms(0, 0, 4, 1024, 2, None) == 1
