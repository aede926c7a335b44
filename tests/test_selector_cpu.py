"""The selector's calibration table on a machine without a GPU: file parsing
and validation, interpolation in (log rows, log time), the choice among
measured candidates, forced paths, pricing a width the table did not measure
from the same plans at the nearest measured widths, the analytic fallback
where the table measured none of the legal plans, and the CREDIT_CALIB
environment variable."""
import json
import math
import os
import subprocess
import sys

import pytest

from wide_reduction_reuse_amd import credit as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def restore_bundled_calibration():
    yield
    C.credit_load_calibration(C.CALIB_PATH if os.path.exists(C.CALIB_PATH) else None)


# two measured candidates for softmax fp32 rows of 4096 columns
ENTRY_A = [0, 0, 4096, 1, 1, 512, 2, 16, -1, 2, 100, 10.0, 1000, 50.0]   # path 1, 512 x 2
ENTRY_B = [0, 0, 4096, 2, 2, 256, 8, 16, 0, 2, 100, 5.0, 1000, 100.0]    # path 2, P = 2, 256 x 8


def _write(tmp_path, table, name="cal.json", **extra):
    doc = {"version": 2, "stream_gbs": 5000.0, "table": table}
    doc.update(extra)
    p = tmp_path / name
    p.write_text(json.dumps(doc))
    return str(p)


def _loglog(r1, t1, r2, t2, r):
    return math.exp(math.log(t1) + (math.log(t2) - math.log(t1)) * (math.log(r) - math.log(r1)) /
                    (math.log(r2) - math.log(r1)))


def test_table_choice_follows_interpolated_times(tmp_path):
    C.credit_load_calibration(_write(tmp_path, [ENTRY_A, ENTRY_B]))
    p = C.credit_select_path("softmax", "f32", 100, 4096)
    assert (p.path, p.split_p, p.block_threads, p.items) == (2, 2, 256, 8)
    p = C.credit_select_path("softmax", "f32", 1000, 4096)
    assert (p.path, p.split_p, p.block_threads, p.items, p.wgs_per_cu) == (1, 1, 512, 2, -1)
    # 300 rows: A = 10 * 5^k, B = 5 * 20^k with k = log(3)/log(10): B is faster
    p = C.credit_select_path("softmax", "f32", 300, 4096)
    assert p.path == 2
    assert p.predicted_us[0] == pytest.approx(_loglog(100, 10, 1000, 50, 300), rel=1e-9)
    assert p.predicted_us[1] == pytest.approx(_loglog(100, 5, 1000, 100, 300), rel=1e-9)
    assert p.predicted_us[2] < 0  # path 3 not measured for this width
    # beyond the measured rows the end segment extends
    p = C.credit_select_path("softmax", "f32", 10000, 4096)
    assert p.path == 1 and p.predicted_us[0] == pytest.approx(_loglog(100, 10, 1000, 50, 10000), rel=1e-9)


def test_forced_paths_use_the_table_and_fall_back(tmp_path):
    C.credit_load_calibration(_write(tmp_path, [ENTRY_A, ENTRY_B]))
    p = C.credit_plan("softmax", "f32", 100, 4096, "single")
    assert (p.path, p.block_threads, p.items) == (1, 512, 2)
    p = C.credit_plan("softmax", "f32", 1000, 4096, "split", 2)
    assert (p.path, p.split_p, p.block_threads, p.items) == (2, 2, 256, 8)
    # P = 4 and path 3 are not in the table: the analytic model plans them
    p = C.credit_plan("softmax", "f32", 1000, 4096, "split", 4)
    assert p.path == 2 and p.split_p == 4
    p = C.credit_plan("softmax", "f32", 1000, 4096, "reread")
    assert p.path == 3


def test_width_whose_plans_were_never_measured_uses_the_analytic_model(tmp_path):
    # at 65536 columns none of the legal plans is one the table measured (at
    # any width), so the analytic model decides, as with no table at all
    C.credit_load_calibration(_write(tmp_path, [ENTRY_A, ENTRY_B]))
    a = C.credit_select_path("softmax", "f32", 1000, 65536).as_dict()
    C.credit_load_calibration(None)
    b = C.credit_select_path("softmax", "f32", 1000, 65536).as_dict()
    # (the predicted times differ: the table's stream rate feeds the model)
    keys = ("path", "split_p", "block_threads", "items", "vec_bytes", "wgs_per_cu")
    assert [a[k] for k in keys] == [b[k] for k in keys]


# the plan of ENTRY_B measured again at 8192 columns
ENTRY_B8 = [0, 0, 8192, 2, 2, 256, 8, 16, 0, 2, 100, 9.0, 1000, 150.0]


def test_width_between_measured_widths_interpolates_the_plan(tmp_path):
    # 6144 columns: split P = 2, 256 x 8 is legal and was measured at 4096 and
    # 8192; each side is read at the rows that move the same bytes, and the two
    # are interpolated in (log cols, log time); path 1's measured tile (512 x 2)
    # cannot hold the row, so only the split plan is priced
    C.credit_load_calibration(_write(tmp_path, [ENTRY_A, ENTRY_B, ENTRY_B8]))
    rows = 500
    p = C.credit_select_path("softmax", "f32", rows, 6144)
    assert (p.path, p.split_p, p.block_threads, p.items) == (2, 2, 256, 8)
    lo = _loglog(100, 5.0, 1000, 100.0, rows * 6144 / 4096)
    hi = _loglog(100, 9.0, 1000, 150.0, rows * 6144 / 8192)
    w = math.log(6144 / 4096) / math.log(2.0)
    assert p.predicted_us[1] == pytest.approx(math.exp((1 - w) * math.log(lo) + w * math.log(hi)), rel=1e-9)
    assert p.predicted_us[0] < 0 and p.predicted_us[2] < 0


def test_width_beyond_the_measured_widths_scales_at_equal_bytes(tmp_path):
    # 12288 columns: the plan was measured below only (4096 and 8192); the
    # nearest width is read at the rows that move the same bytes
    C.credit_load_calibration(_write(tmp_path, [ENTRY_A, ENTRY_B, ENTRY_B8]))
    p = C.credit_plan("softmax", "f32", 300, 12288, "split", 2)
    assert (p.path, p.split_p, p.block_threads, p.items) == (2, 2, 256, 8)
    assert p.predicted_us[1] == pytest.approx(_loglog(100, 9.0, 1000, 150.0, 300 * 12288 / 8192), rel=1e-9)


@pytest.mark.parametrize("bad", [
    [0, 0, 4096, 1, 1, 512, 2, 16, -1, 2, 1000, 10.0, 100, 50.0],   # rows not ascending
    [0, 0, 4096, 4, 1, 512, 2, 16, -1, 2, 100, 10.0, 1000, 50.0],   # no path 4
    [0, 0, 4096, 1, 1, 512, 2, 16, -1, 2, 100, 10.0, 1000],         # a point is missing
    [0, 0, 4096, 1, 1, 512, 2, 16, -1, 2, 100, -1.0, 1000, 50.0],   # non-positive time
    [6, 0, 4096, 1, 1, 512, 2, 16, -1, 2, 100, 10.0, 1000, 50.0],   # no op 6
    [4, 2, 4096, 1, 1, 512, 2, 16, -1, 2, 100, 10.0, 1000, 50.0],   # no dtype 2
    [0, 0, 4096, 1, 1, 512, 2, 16, -1],                             # header cut short
])
def test_malformed_tables_are_refused_and_the_previous_one_stays(tmp_path, bad):
    C.credit_load_calibration(_write(tmp_path, [ENTRY_A, ENTRY_B], "good.json"))
    assert C.lib().credit_load_calibration(_write(tmp_path, [ENTRY_A, bad], "bad.json").encode()) == 6
    assert C.credit_select_path("softmax", "f32", 100, 4096).path == 2


def test_bundled_calibration_loads_and_chooses_the_one_read_paths():
    assert os.path.exists(C.CALIB_PATH)
    C.credit_load_calibration(C.CALIB_PATH)
    p = C.credit_select_path("softmax", "f32", 256, 262144)
    assert p.path == 2 and p.split_p in (2, 4, 8)  # one CU cannot hold a 1 MiB row
    for op, dt, rows, cols in [("softmax", "f32", 64, 4096), ("layernorm", "bf16", 4096, 8192),
                               ("rmsnorm", "bf16", 1024, 65536)]:
        p = C.credit_select_path(op, dt, rows, cols)
        assert p.path in (1, 2, 3) and p.predicted_us[p.path - 1] > 0


def test_calibration_from_environment(tmp_path):
    path = _write(tmp_path, [ENTRY_A, ENTRY_B])
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from wide_reduction_reuse_amd import credit as C\n"
            "p = C.credit_select_path('softmax', 'f32', 100, 4096)\n"
            "print(p.path, p.split_p, p.block_threads, p.items)\n" % ROOT)
    env = dict(os.environ, CREDIT_CALIB=path)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["2", "2", "256", "8"]


def test_crossover_width_report():
    # a series of widths where splitting is measured to pay from 16384 on;
    # the report finds the first width from which the split stays ahead
    from wide_reduction_reuse_amd import selector_eval as E
    records, rows = [], []
    for cols, meas, pred in [(4096, False, False), (8192, True, False), (16384, True, True), (32768, True, True)]:
        records.append({"op": "softmax", "dtype": "f32", "rows": 64, "cols": cols, "workload": "next_x"})
        rows.append({"split_ok": meas == pred, "split_meas": meas, "split_pred": pred})
    rep = E.crossover(records, rows)
    assert len(rep) == 1
    assert rep[0]["measured"] == 8192 and rep[0]["predicted"] == 16384 and rep[0]["steps_off"] == 1
    # a split that never pays has no crossover
    rows2 = [dict(r, split_meas=False, split_pred=False) for r in rows]
    rep = E.crossover(records, rows2)
    assert rep[0]["measured"] is None and rep[0]["steps_off"] == 0


def test_peak_bandwidth_ablation_changes_only_the_rate(tmp_path):
    # the ablation prices the stream at the device peak: every estimate can
    # only get faster than at a lower achieved rate
    C.credit_load_calibration(_write(tmp_path, [], "achieved.json"))
    slow = C.credit_select_path("softmax", "f32", 4096, 4096).predicted_us[0]
    p = tmp_path / "peak.json"
    p.write_text(json.dumps({"version": 2, "stream_gbs": 1000.0, "model_peak_bandwidth": 1}))
    C.credit_load_calibration(str(p))
    fast = C.credit_select_path("softmax", "f32", 4096, 4096).predicted_us[0]
    assert fast < slow


def test_control_fit_recovers_launch_and_per_wave_cost():
    from wide_reduction_reuse_amd.ctrlbench import fit_line
    a, b = fit_line([1, 2, 4, 8, 16], [3.0 + 0.5 * w for w in (1, 2, 4, 8, 16)])
    assert abs(a - 3.0) < 1e-12 and abs(b - 0.5) < 1e-12


def test_calibration_merges_repeated_timings_by_geometric_mean():
    from wide_reduction_reuse_amd import calibrate as K
    plan = {"path": 1, "split_p": 1, "block_threads": 512, "items": 2, "vec_bytes": 16, "wgs_per_cu": -1}

    def rec(rows, ms):
        return {"op": "softmax", "dtype": "f32", "rows": rows, "cols": 4096,
                "candidates": [{"plan": plan, "median_ms": ms}]}
    records = [rec(100, 0.010), rec(1000, 0.050), rec(100, 0.040)]  # 100 rows timed twice
    table = K.build_table(records)
    assert len(table) == 1
    row = table[0]
    assert row[:10] == [0, 0, 4096, 1, 1, 512, 2, 0, 16, -1] and row[10] == 2
    assert row[11] == 100 and row[12] == pytest.approx(math.sqrt(10.0 * 40.0), rel=1e-4)
    assert row[13] == 1000 and row[14] == pytest.approx(50.0)
    assert K.unique_shapes(records) == 2


def test_calibration_extension_keeps_base_rows_and_merges_shared_ones():
    from wide_reduction_reuse_amd import calibrate as K
    base = [[0, 0, 4096, 1, 1, 512, 2, 0, 16, -1, 2, 100, 10.0, 1000, 50.0],
            [2, 1, 8192, 1, 1, 64, 16, 0, 16, 0, 1, 64, 5.0]]
    new = [[0, 0, 4096, 1, 1, 512, 2, 0, 16, -1, 2, 100, 40.0, 4000, 190.0],   # same plan: 100 rows again, 4000 new
           [0, 1, 1026, 1, 1, 256, 4, 0, 16, -1, 1, 8192, 7.0],               # a plan the base never measured
           [0, 0, 4096, 1, 1, 512, 2, 8, 16, -1, 1, 100, 9.0]]                # the same tile with an LDS part
    t = K.merge_tables(base, new)
    assert [r[:10] for r in t] == sorted([r[:10] for r in base] + [new[1][:10], new[2][:10]])
    shared = next(r for r in t if r[:3] == [0, 0, 4096] and r[7] == 0)
    assert shared[10] == 3 and shared[11] == 100 and shared[12] == pytest.approx(20.0)
    assert shared[13:] == [1000, 50.0, 4000, 190.0]
    # version 2 rows (no LDS column) read as register tiles
    assert K.upgrade_rows({"version": 2, "table": [base[0][:7] + base[0][8:]]}) == [base[0]]
    assert next(r for r in t if r[:3] == [2, 1, 8192]) == base[1]
    assert next(r for r in t if r[:3] == [0, 1, 1026]) == new[1]


def test_calibration_extension_drops_plans_the_library_no_longer_offers():
    # an odd-length bf16 softmax row is held as 16-byte vectors now: a table
    # row of its one-element held tile is stale, its reread row and the
    # 16-byte held row are offered
    from wide_reduction_reuse_amd import calibrate as K
    stale = [0, 1, 50257, 1, 1, 1024, 32, 0, 2, -1, 1, 2670, 250.0]
    held = [0, 1, 50257, 1, 1, 512, 16, 0, 16, -1, 1, 2670, 120.0]
    reread = [0, 1, 50257, 3, 1, 256, 8, 0, 2, 0, 1, 2670, 320.0]
    assert not K.offered(stale)
    assert K.offered(held) and K.offered(reread)
    # an LDS part is offered only for rows of whole 16-byte vectors
    assert not K.offered(held[:7] + [8] + held[8:])


def test_width_missing_a_legal_held_path_is_priced_from_the_neighbours(tmp_path):
    # the table timed only the reread path at 4096 columns (as a table timed
    # on a kernel set without held tiles for such rows would): it cannot weigh
    # paths 1 and 2 there, so the neighbours (here none) and the analytic
    # model decide, not the one timed plan however fast it was
    reread_only = [0, 0, 4096, 3, 1, 256, 8, 16, 0, 2, 100, 0.1, 1000, 0.5]
    C.credit_load_calibration(_write(tmp_path, [reread_only]))
    p = C.credit_select_path("softmax", "f32", 1000, 4096)
    assert p.path != 3
    # forced to the reread path, the table's plan is used
    assert C.credit_plan("softmax", "f32", 1000, 4096, "reread").path == 3


def test_table_plans_that_no_longer_hold_the_row_are_passed_over(tmp_path):
    # 4100 fp32 columns are held shifted (up to 48 bytes in front): 1028
    # vectors, which a 1024 x 1 tile (1024 vectors) does not hold, though a
    # table timed before rows were shifted could list it; it is passed over
    # for the table's other plan
    stale = [0, 0, 4100, 1, 1, 1024, 1, 16, -1, 2, 100, 1.0, 1000, 5.0]
    other = [0, 0, 4100, 1, 1, 512, 4, 16, -1, 2, 100, 50.0, 1000, 500.0]
    split = [0, 0, 4100, 2, 2, 256, 4, 16, 0, 2, 100, 60.0, 1000, 600.0]
    C.credit_load_calibration(_write(tmp_path, [stale, other, split]))
    p = C.credit_select_path("softmax", "f32", 1000, 4100)
    assert (p.path, p.block_threads, p.items) == (1, 512, 4)
