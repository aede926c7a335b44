"""The LDS tier on the host: legality of held rows by registers plus LDS
(the Eq. 3 analogue of the CREDIT paper, Sec. III-B), which tiles the
planner offers, and the plan checks the library makes before any launch."""
import os

import pytest

from wide_reduction_reuse_amd import credit as C


@pytest.fixture(autouse=True)
def analytic_model_only():
    C.credit_load_calibration(None)
    yield
    C.credit_load_calibration(C.CALIB_PATH if os.path.exists(C.CALIB_PATH) else None)


def _plan(op, dt, rows, cols, path, p=0):
    try:
        return C.credit_plan(op, dt, rows, cols, path, p)
    except C.CreditError as e:
        assert e.status == 4, e.status
        return None


@pytest.mark.parametrize("op,dt,reg_max,lds_max", [
    # widest row of whole 16-byte vectors path 1 holds in registers alone, and with the LDS tier
    ("softmax", "f32", 65536, 98304), ("softmax", "bf16", 131072, 196608),
    ("rmsnorm", "f32", 65536, 98304), ("quantize_int8", "bf16", 131072, 196608),
    ("softmax_bwd", "f32", 32768, 49152), ("layernorm_bwd", "f32", 32768, 49152),
    ("layernorm", "f32", 65536, 65536),  # LayerNorm's 1024-thread LDS tile spilled: none built
])
def test_path1_legality_registers_plus_lds(op, dt, reg_max, lds_max):
    epv = 4 if dt == "f32" else 8
    p = _plan(op, dt, 64, reg_max, "single")
    assert p is not None and p.lds_items == 0  # registers hold it: no LDS part
    if lds_max > reg_max:
        p = _plan(op, dt, 64, reg_max + epv, "single")
        assert p is not None and p.lds_items > 0
        assert p.block_threads * p.items < (reg_max + epv) // epv <= p.block_threads * (p.items + p.lds_items)
        p = _plan(op, dt, 64, lds_max, "single")
        assert p is not None and p.lds_items > 0
    assert _plan(op, dt, 64, lds_max + epv, "single") is None


def test_rows_not_of_whole_vectors_get_no_lds_part():
    # 98302 fp32 columns end in a partial 16-byte vector: registers only, and
    # no register tile holds 24576 vectors
    assert _plan("softmax", "f32", 64, 98302, "single") is None
    assert _plan("softmax", "f32", 64, 98304, "single").lds_items == 8


def test_split_slices_use_the_lds_tier_only_past_registers():
    # 196608 fp32 columns: P = 2 slices of 98304 need the LDS tier, P = 4 do not
    p2 = _plan("softmax", "f32", 64, 196608, "split", 2)
    p4 = _plan("softmax", "f32", 64, 196608, "split", 4)
    assert p2.lds_items == 8 and p2.block_threads == 1024
    assert p4.lds_items == 0
    assert _plan("softmax", "f32", 64, 262144, "split", 2) is None  # 1 MiB halves: still too wide


def test_enumeration_offers_lds_tiles_between_register_and_lds_capacity():
    plans = [p.as_dict() for p in C.credit_enumerate_plans("softmax", "f32", 256, 81920)]
    lds = [p for p in plans if p["lds_items"]]
    assert {(p["path"], p["block_threads"], p["items"], p["lds_items"]) for p in lds} >= {(1, 1024, 16, 8)}
    assert {p["wgs_per_cu"] for p in lds if p["path"] == 1} == {0, -1}
    # where registers alone hold the row, no LDS tile is offered for it
    assert not [p for p in C.credit_enumerate_plans("softmax", "f32", 256, 65536)
                if p.lds_items and p.path == 1]
    # and none for rows that are not whole 16-byte vectors
    assert not [p for p in C.credit_enumerate_plans("softmax", "f32", 256, 81918) if p.lds_items]


def test_plan_checks_before_launch():
    # resolve the plan on the host; errors come back before any HIP call
    # (credit_occupancy would query the device next, which fails here)
    L = C.lib()
    import ctypes
    n = ctypes.c_int32()

    def status(cols, plan):
        return L.credit_occupancy(0, 0, cols, ctypes.byref(plan), ctypes.byref(n))
    mk = C.Plan.make
    assert status(98304, mk(1, 1, 1024, 16, 16, -1, lds_items=-1)) == 1          # negative
    assert status(98304 + 4, mk(1, 1, 1024, 16, 16, -1, lds_items=8)) == 4        # past the LDS part
    assert status(98302, mk(1, 1, 1024, 16, 16, -1, lds_items=8)) == 4            # partial last vector
    assert status(8192, mk(1, 1, 64, 16, 16, -1, lds_items=8)) == 4               # wave tiles have none
    assert status(98304, mk(3, 1, 1024, 4, 16, 0, lds_items=8)) == 4              # nor the reread path
    assert status(98304, mk(1, 1, 1024, 16, 16, -1, lds_items=4)) == 2            # not compiled
    assert status(98304, mk(1, 1, 1024, 16, 16, -1, lds_items=8)) not in (1, 2, 4)  # legal: the device query
