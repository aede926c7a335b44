"""The model-constant fit (model_fit.py) on the CPU: it recovers constants
from timings the library's own model produced under known constants, keeps
the occupancy it is given, and writes a calibration the library loads."""
import json
import os

import pytest

from wide_reduction_reuse_amd import credit as C
from wide_reduction_reuse_amd import model_fit as F


@pytest.fixture(autouse=True)
def restore_bundled_calibration():
    yield
    C.credit_load_calibration(C.CALIB_PATH if os.path.exists(C.CALIB_PATH) else None)


SHAPES = [("softmax", "f32", r, c) for r, c in [(64, 4096), (4096, 4096), (256, 16384), (32, 65536), (2048, 65536),
                                                 (16, 262144), (256, 262144), (1024, 131072)]] + \
         [("rmsnorm", "bf16", r, c) for r, c in [(8192, 2048), (64, 65536), (1024, 65536), (128, 524288)]] + \
         [("layernorm", "f32", r, c) for r, c in [(1024, 8192), (64, 65536), (512, 131072)]]


def _synthetic(consts):
    """Records whose every candidate's time is the model's prediction under
    `consts` (an exact fit exists)."""
    ev = F.Evaluator(C, [], [])
    ev.load(consts)
    recs = []
    for op, dt, rows, cols in SHAPES:
        cands = []
        for p in C.credit_enumerate_plans(op, dt, rows, cols):
            d = p.as_dict()
            us = d["predicted_us"][d["path"] - 1]
            plan = {k: d[k] for k in ("path", "split_p", "block_threads", "items", "vec_bytes", "wgs_per_cu",
                                      "lds_items")}
            cands.append({"plan": plan, "median_ms": us / 1e3})
        recs.append({"workload": "syn", "op": op, "dtype": dt, "rows": rows, "cols": cols, "candidates": cands})
    return recs


def test_fit_recovers_the_timings_of_known_constants():
    truth = dict(F.DEFAULTS)
    truth.update(bw_gbs=4000.0, launch_us=5.0, exch_us=2.0, split_launch_us=6.0, l0_us=3.0, owner_gbs=30.0)
    recs = _synthetic(truth)
    logs = []
    got = F.fit(C, recs, [], start=dict(F.DEFAULTS), log=logs.append)
    assert len(logs) == 2
    # both stages end with (near) zero log error on the timings they fit
    for line in logs:
        assert float(line.split("->")[1]) < 0.02, line
    # the constants every plan's time depends on come back
    assert got["launch_us"] == pytest.approx(5.0, rel=0.1)
    assert got["bw_gbs"] == pytest.approx(4000.0, rel=0.1)
    assert got["word_gbs"] == F.DEFAULTS["word_gbs"]  # not fitted


def test_row_kind_matches_the_kernel_families():
    C.credit_load_calibration(None)
    assert F.row_kind("softmax", "f32", 4096) == 0
    assert F.row_kind("softmax", "f32", 30001) == 2        # not a multiple of 64 bytes: shifted
    assert F.row_kind("softmax", "f32", 4100) == 2         # 16-byte multiple, not 64: shifted too
    assert F.row_kind("softmax", "f32", 1004) == 2
    assert F.row_kind("softmax", "bf16", 20002) == 2
    assert F.row_kind("softmax", "bf16", 50257) == 2
    assert F.row_kind("quantize_int8", "f32", 1001) == 2
    assert F.row_kind("softmax_bwd", "f32", 48) == 0       # 192 bytes: whole lines
    assert F.row_kind("rmsnorm", "f32", 30001) == 2        # parameters realigned per row
    assert F.row_kind("layernorm", "bf16", 20002) == 1     # LayerNorm shifts odd bf16 rows only
    assert F.row_kind("layernorm", "bf16", 20001) == 2
    assert F.row_kind("layernorm", "f32", 1004) == 0
    assert F.row_kind("rmsnorm", "bf16", 50257) == 2
    assert F.row_kind("layernorm_bwd", "f32", 30001) == 1  # a partial last vector
    assert F.row_kind("layernorm_bwd", "f32", 4100) == 2   # 16-byte multiple, not a 64-byte one: shifted
    assert F.row_kind("layernorm_bwd", "f32", 4096) == 0
    # its split slices keep their parameters and do not shift
    assert F.row_kind("layernorm_bwd", "f32", 30001, 2) == 1
    assert F.row_kind("layernorm_bwd", "f32", 4100, 2) == 0
    assert F.row_kind("softmax", "f32", 4100, 2) == 2
    assert F.row_kind("layernorm_bwd", "bf16", 20002) == 2  # shifted raw bf16 tiles on path 1
    assert F.row_kind("layernorm_bwd", "bf16", 1000) == 0   # whole 16-byte vectors: held as they are
    assert F.row_kind("layernorm_bwd", "bf16", 20001, 2) == 0  # 2-byte accesses on path 2
    # the library holds kind-2 widths with room for the shift, kind-1 widths without
    assert C.credit_plan("softmax", "f32", 64, 4100, "single").block_threads * \
        C.credit_plan("softmax", "f32", 64, 4100, "single").items * 4 >= 4100 + 12
    assert C.credit_plan("layernorm_bwd", "f32", 64, 1022, "single").block_threads * \
        C.credit_plan("layernorm_bwd", "f32", 64, 1022, "single").items * 4 >= 1022


def test_occupancy_table_and_written_calibration_load(tmp_path):
    C.credit_load_calibration(None)
    rec = {"workload": "w", "op": "softmax", "dtype": "f32", "rows": 64, "cols": 30001, "candidates": [
        {"plan": {"path": 1, "split_p": 1, "block_threads": 512, "items": 4, "vec_bytes": 16, "wgs_per_cu": -1},
         "median_ms": 0.01, "occupancy": 3},
        {"plan": {"path": 1, "split_p": 1, "block_threads": 64, "items": 16, "vec_bytes": 16, "wgs_per_cu": -1},
         "median_ms": 0.01, "occupancy": 5},
        {"plan": {"path": 2, "split_p": 4, "block_threads": 256, "items": 2, "vec_bytes": 16, "wgs_per_cu": 0},
         "median_ms": 0.01, "occupancy": 6},
        {"plan": {"path": 3, "split_p": 1, "block_threads": 512, "items": 4, "vec_bytes": 4, "wgs_per_cu": 0},
         "median_ms": 0.01, "occupancy": 4}]}
    occ = F.occupancy_table(C, [rec])
    assert occ == [[0, 0, 1, 64, 16, 16, 2, 0, 5], [0, 0, 2, 512, 4, 16, 2, 0, 3], [0, 0, 3, 256, 2, 16, 2, 0, 6],
                   [0, 0, 4, 512, 4, 4, 0, 0, 4]]
    src = tmp_path / "in.jsonl"
    src.write_text(json.dumps(rec) + "\n")
    out = tmp_path / "cal.json"
    # a fit on one shape is meaningless; the point is the file it writes
    F.main([str(src), "--out", str(out)])
    doc = json.loads(out.read_text())
    assert doc["occupancy"] == occ and set(F.DEFAULTS) <= set(doc["model"])
    C.credit_load_calibration(str(out))
