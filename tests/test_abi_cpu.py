"""The C-ABI library on a machine without a GPU: it loads, exports every entry
point include/credit.h declares, validates arguments before touching the
device, and its host-only selector and calibration loader work."""
import ctypes
import json
import os
import re

import pytest

from wide_reduction_reuse_amd import credit as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "credit.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(credit_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = C.lib()
    names = _declared()
    assert "credit_softmax" in names and "credit_select_path" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(C.EXPORTED)
    assert C.credit_version() == 100


def test_status_strings():
    for code in range(9):
        assert C.credit_status_str(code) and C.credit_status_str(code) != "unknown status"
    assert C.credit_status_str(99) == "unknown status"


# Fake but 16-byte-aligned device addresses: validation must reject the call
# before any HIP call could dereference them.
A = ctypes.c_void_p(0x7F0000000000)
B = ctypes.c_void_p(0x7F0000100000)
G = ctypes.c_void_p(0x7F0000200000)
MIS = ctypes.c_void_p(0x7F0000000004)


def _sm(x=A, y=B, rows=4, cols=64, dt=0, path=0, p=0):
    return C.lib().credit_softmax(x, y, rows, cols, dt, path, p, None)


def _ln(x=A, g=G, b=G, y=B, rows=4, cols=64, eps=1e-5, dt=0, path=0, p=0):
    return C.lib().credit_layernorm(x, g, b, y, rows, cols, eps, dt, path, p, None)


def _rms(x=A, g=G, y=B, rows=4, cols=64, eps=1e-6, dt=0, path=0, p=0):
    return C.lib().credit_rmsnorm(x, g, y, rows, cols, eps, dt, path, p, None)


def _smb(x=A, dy=G, dx=B, rows=4, cols=64, dt=0, path=0, p=0):
    return C.lib().credit_softmax_backward(x, dy, dx, rows, cols, dt, path, p, None)


def _lnb(x=A, dy=G, g=G, dx=B, rows=4, cols=64, eps=1e-5, dt=0, path=0, p=0):
    return C.lib().credit_layernorm_backward(x, dy, g, dx, rows, cols, eps, dt, path, p, None)


S4 = ctypes.c_void_p(0x7F0000300004)  # 4-byte aligned: enough for the scale vector


def _q(x=A, q=B, s=S4, rows=4, cols=64, dt=0, path=0, p=0):
    return C.lib().credit_quantize_int8(x, q, s, rows, cols, dt, path, p, None)


@pytest.mark.parametrize("call,status", [
    (lambda: _sm(x=None), 1), (lambda: _sm(y=None), 1), (lambda: _sm(cols=0), 1),
    (lambda: _sm(rows=-1), 1), (lambda: _sm(dt=2), 1), (lambda: _sm(path=4), 1),
    (lambda: _sm(path=2, p=3), 1), (lambda: _sm(path=1, p=4), 1), (lambda: _sm(x=MIS), 3),
    (lambda: _sm(y=MIS), 3), (lambda: _sm(rows=1 << 40, cols=1 << 40), 1),
    (lambda: _ln(g=None), 1), (lambda: _ln(b=None), 1), (lambda: _ln(eps=-1.0), 1),
    (lambda: _ln(eps=float("nan")), 1), (lambda: _ln(eps=float("inf")), 1), (lambda: _ln(b=MIS), 3),
    (lambda: _rms(g=None), 1), (lambda: _rms(eps=-1e-6), 1), (lambda: _rms(g=MIS), 3),
    (lambda: _smb(dy=None), 1), (lambda: _smb(dx=None), 1), (lambda: _smb(dy=MIS), 3), (lambda: _smb(dt=2), 1),
    (lambda: _lnb(dy=None), 1), (lambda: _lnb(g=None), 1), (lambda: _lnb(eps=-1.0), 1),
    (lambda: _lnb(dy=MIS), 3), (lambda: _lnb(dt=2), 1),
    (lambda: _q(q=None), 1), (lambda: _q(s=None), 1), (lambda: _q(x=MIS), 3),
    (lambda: _q(s=ctypes.c_void_p(0x7F0000300002)), 3), (lambda: _q(cols=0), 1),
])
def test_invalid_arguments_rejected_before_launch(call, status):
    assert call() == status


def test_rows_zero_is_a_noop_without_device():
    assert _sm(rows=0) == 0
    assert _sm(x=None, y=None, rows=0) == 0
    assert _ln(rows=0) == 0
    assert _rms(rows=0) == 0
    assert _smb(rows=0) == 0 and _lnb(rows=0) == 0 and _q(rows=0) == 0


def test_forced_path_that_cannot_hold_the_row_is_refused():
    # path 1 cannot hold a 1 MiB fp32 row; P=2 cannot either
    assert _sm(cols=262144, path=1) == 4
    assert _sm(cols=262144, path=2, p=2) == 4
    # too narrow to split eight ways (the last slice would be empty)
    assert _sm(cols=8, path=2, p=8) == 4


def _ops(**kw):
    o = C.Operands()
    for k, v in kw.items():
        setattr(o, k, v.value if isinstance(v, ctypes.c_void_p) else v)
    return ctypes.byref(o)


def test_run_plan_validation():
    L = C.lib()
    sm = _ops(x=A, y=B)
    plan = C.Plan.make(C.PATH_SINGLE_WG, 1, 64, 3, 16)  # no such tile
    assert L.credit_run_plan(0, sm, 4, 64, 0.0, 0, ctypes.byref(plan), None) == 2
    plan = C.Plan.make(C.PATH_SINGLE_WG, 1, 64, 1, 16)  # holds 64 vectors = 256 fp32 only
    assert L.credit_run_plan(0, sm, 4, 1024, 0.0, 0, ctypes.byref(plan), None) == 4
    plan = C.Plan.make(C.PATH_SPLIT_ROW, 3, 256, 8, 16)  # P must be 2, 4 or 8
    assert L.credit_run_plan(0, sm, 4, 4096, 0.0, 0, ctypes.byref(plan), None) == 4
    assert L.credit_run_plan(0, sm, 4, 4096, 0.0, 0, None, None) == 1
    assert L.credit_run_plan(0, None, 4, 4096, 0.0, 0, ctypes.byref(plan), None) == 1
    plan = C.Plan.make(C.PATH_REREAD, 1, 256, 4, 4)  # vec_bytes does not match the row
    assert L.credit_run_plan(0, sm, 4, 4096, 0.0, 0, ctypes.byref(plan), None) == 4
    # each operator requires its own operands
    plan = C.Plan.make(C.PATH_SINGLE_WG, 1, 64, 1, 16)
    assert L.credit_run_plan(3, sm, 4, 64, 0.0, 0, ctypes.byref(plan), None) == 1        # dy missing
    assert L.credit_run_plan(4, _ops(x=A, dy=G, y=B), 4, 64, 1e-5, 0, ctypes.byref(plan), None) == 1  # gamma
    assert L.credit_run_plan(5, sm, 4, 64, 0.0, 0, ctypes.byref(plan), None) == 1        # scale missing
    assert L.credit_run_plan(6, sm, 4, 64, 0.0, 0, ctypes.byref(plan), None) == 1        # no such operator
    # a spilling tile the registry leaves out is not compiled for that operator
    plan = C.Plan.make(C.PATH_SINGLE_WG, 1, 1024, 8, 16)
    assert L.credit_run_plan(4, _ops(x=A, dy=G, gamma=G, y=B), 4, 32768, 1e-5, 0, ctypes.byref(plan), None) == 2


def test_run_plan_timed_validation():
    L = C.lib()
    E1, E2 = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)
    plan = C.Plan.make(C.PATH_SINGLE_WG, 1, 64, 1, 16)
    sm = _ops(x=A, y=B)
    # both events are required, and an empty launch cannot be timed
    assert L.credit_run_plan_timed(0, sm, 4, 64, 0.0, 0, ctypes.byref(plan), None, E2, None) == 1
    assert L.credit_run_plan_timed(0, sm, 4, 64, 0.0, 0, ctypes.byref(plan), E1, None, None) == 1
    assert L.credit_run_plan_timed(0, sm, 0, 64, 0.0, 0, ctypes.byref(plan), E1, E2, None) == 1
    assert L.credit_run_plan_timed(0, _ops(x=MIS, y=B), 4, 64, 0.0, 0, ctypes.byref(plan), E1, E2, None) == 3
    assert L.credit_run_plan_timed(0, sm, 4, 1024, 0.0, 0, ctypes.byref(plan), E1, E2, None) == 4


def test_misc_entry_points_validate():
    L = C.lib()
    assert L.credit_copy(None, B, 16, None, None, None) == 1
    assert L.credit_copy(A, B, 15, None, None, None) == 1
    assert L.credit_copy(MIS, B, 16, None, None, None) == 3
    assert L.credit_copy(A, B, 0, None, None, None) == 0
    assert L.credit_flush(None, 16, None) == 1
    assert L.credit_flush(A, 0, None) == 0
    plan = C.Plan.make(C.PATH_SINGLE_WG, 1, 64, 1, 16)
    assert L.credit_control(0, 4, 64, 0, ctypes.byref(plan), None, None, None) == 1  # control needs a split plan
    assert L.credit_control(0, 4, 64, 0, None, None, None, None) == 1
    split = C.Plan.make(C.PATH_SPLIT_ROW, 2, 256, 8, 16)
    assert L.credit_control(0, 0, 4096, 0, ctypes.byref(split), None, None, None) == 0  # rows = 0: no-op
    split_lds = C.Plan.make(C.PATH_SPLIT_ROW, 2, 1024, 16, 16, lds_items=8)
    assert L.credit_control(0, 4, 4096, 0, ctypes.byref(split_lds), None, None, None) == 2  # control twins: registers only


def test_selector_legality_on_cpu():
    # rows of one MiB (fp32 262144) exceed one CU: path 1 illegal, path 2 chosen
    p = C.credit_select_path("softmax", "f32", 256, 262144)
    assert p.predicted_us[0] < 0 and p.predicted_us[1] > 0 and p.predicted_us[2] > 0
    assert p.path in (C.PATH_SPLIT_ROW, C.PATH_REREAD)
    # a 16 KiB row fits one owner
    p = C.credit_select_path("layernorm", "bf16", 4096, 8192)
    assert p.predicted_us[0] > 0
    # rows whose byte length is not a multiple of 16 use one-element accesses
    p = C.credit_select_path("rmsnorm", "bf16", 10, 1001)
    assert p.vec_bytes == 2
    assert C.lib().credit_select_path(0, 0, 1, 1, None) == 1
    assert C.lib().credit_select_path(6, 0, 1, 1, ctypes.byref(C.Plan())) == 1
    assert C.lib().credit_select_path(4, 2, 1, 1, ctypes.byref(C.Plan())) == 1  # no such dtype
    assert C.lib().credit_select_path(4, 1, 1, 1, ctypes.byref(C.Plan())) == 0  # LayerNorm backward bf16


def test_partial_rows_are_held_as_16_byte_vectors():
    # byte length a multiple of 4 but not of 16, LayerNorm and fp32
    # LayerNorm backward: paths 1 and 2 hold the row as 16-byte vectors from
    # its first byte (the last partial) and reread it by element
    L = C.lib()
    for op, dt, cols in [("layernorm", "bf16", 1002), ("layernorm", "f32", 3), ("layernorm_bwd", "f32", 1001)]:
        p = C.credit_plan(op, dt, 64, cols, "single")
        assert p.vec_bytes == 16
        assert C.credit_plan(op, dt, 64, cols, "reread").vec_bytes == 16 // (4 if dt == "f32" else 8)
        # the one-element held tile of that width is refused for such rows
        plan = C.Plan.make(C.PATH_SINGLE_WG, 1, p.block_threads, p.items, 4 if dt == "f32" else 2)
        assert L.credit_run_plan(C.OPS[op], _ops(x=A, dy=G, gamma=G, beta=G, y=B), 4, cols, 1e-5,
                                 C.DTYPES[dt], ctypes.byref(plan), None) == 4
    assert C.credit_plan("layernorm_bwd", "f32", 64, 100003, "split", 8).vec_bytes == 16
    # odd-length bf16 rows of LayerNorm backward: shifted on the single path,
    # read by element on the reread path
    assert C.credit_plan("layernorm_bwd", "bf16", 64, 1001, "single").vec_bytes == 16
    assert C.credit_plan("layernorm_bwd", "bf16", 64, 100001, "reread").vec_bytes == 2


def _max_shift_bytes(cols, eb):
    """The most bytes of the previous row in front of any row of a tensor with
    16-byte aligned base, held from the 64-byte line below its start: brute
    force over the base's offset and enough rows to cycle through every start."""
    return max((base + r * cols * eb) % 64 for base in (0, 16, 32, 48) for r in range(0, 65))


def test_shifted_rows_are_held_from_the_line_below():
    # rows whose byte length is not a multiple of 64, of softmax, softmax
    # backward, the quantizer, RMSNorm, LayerNorm's odd-length bf16 rows, and
    # fp32 LayerNorm backward's rows of whole 16-byte vectors (single path):
    # paths 1 and 2 hold them as 16-byte vectors from the 64-byte line below
    # each row's start, so a tile must hold the row plus the largest such
    # offset; the reread path reads them by element (or by 16-byte vector
    # when the byte length is a multiple of 16)
    L = C.lib()
    cases = [("softmax", "f32", 1001), ("softmax", "f32", 1004), ("softmax", "f32", 4100), ("softmax", "f32", 5001),
             ("softmax", "bf16", 1), ("softmax", "bf16", 1001), ("softmax", "bf16", 50257),
             ("softmax", "bf16", 50264), ("softmax_bwd", "bf16", 30001), ("softmax_bwd", "f32", 30006),
             ("quantize_int8", "f32", 1001), ("quantize_int8", "bf16", 1001), ("quantize_int8", "f32", 4100),
             ("layernorm", "bf16", 1001), ("layernorm", "bf16", 50257), ("rmsnorm", "f32", 3),
             ("rmsnorm", "bf16", 50257), ("rmsnorm", "f32", 30001), ("layernorm_bwd", "f32", 100),
             ("layernorm_bwd", "f32", 4100), ("layernorm_bwd", "f32", 12292), ("layernorm_bwd", "bf16", 1001),
             ("layernorm_bwd", "bf16", 20002), ("layernorm_bwd", "bf16", 4100)]
    for op, dt, cols in cases:
        eb = 4 if dt == "f32" else 2
        p = C.credit_plan(op, dt, 64, cols, "single")
        assert p.vec_bytes == 16, (op, dt, cols)
        span = cols * eb + _max_shift_bytes(cols, eb)
        assert p.block_threads * p.items * 16 >= span, (op, dt, cols)
        rvb = 16 if (cols * eb) % 16 == 0 else eb
        assert C.credit_plan(op, dt, 64, cols, "reread").vec_bytes == rvb
        if rvb != 16:
            plan = C.Plan.make(C.PATH_SINGLE_WG, 1, p.block_threads, p.items, eb)
            assert L.credit_run_plan(C.OPS[op], _ops(x=A, dy=G, gamma=G, beta=G, y=B, row_out=G), 4, cols, 1e-5,
                                     C.DTYPES[dt], ctypes.byref(plan), None) == 4
    # a tile that holds the row but not the row plus its largest offset is
    # refused: 4100 fp32 elements (1025 vectors) plus up to 48 bytes need
    # 1028 vectors; 1024 x 1 holds 1024
    small = C.Plan.make(C.PATH_SINGLE_WG, 1, 1024, 1, 16)
    assert L.credit_run_plan(C.OPS["softmax"], _ops(x=A, y=B), 4, 4100, 0.0, C.DTYPES["f32"],
                             ctypes.byref(small), None) == 4
    assert C.credit_plan("softmax", "bf16", 64, 100003, "split", 8).vec_bytes == 16
    # rows of whole 64-byte lines are held as they are
    for op, dt, cols in [("softmax", "f32", 1024), ("quantize_int8", "bf16", 4096), ("softmax_bwd", "f32", 48)]:
        p = C.credit_plan(op, dt, 64, cols, "single")
        assert p.vec_bytes == 16 and p.block_threads * p.items * 16 >= cols * (4 if dt == "f32" else 2)


def test_selector_legality_of_the_further_workloads():
    # x and dy held: path 1 holds at most 32768 fp32 columns (two inputs)
    for op in ("softmax_bwd", "layernorm_bwd"):
        assert C.credit_select_path(op, "f32", 4096, 32768).predicted_us[0] > 0
        p = C.credit_select_path(op, "f32", 4096, 65536)
        assert p.predicted_us[0] < 0 and p.path in (C.PATH_SPLIT_ROW, C.PATH_REREAD)
        with pytest.raises(C.CreditError) as ei:
            C.credit_plan(op, "f32", 4096, 65536, "single")
        assert ei.value.status == 4
    # the quantizer holds one fp32 input: 65536 columns fit one workgroup
    assert C.credit_select_path("quantize_int8", "f32", 4096, 65536).predicted_us[0] > 0
    # every enumerated plan of a two-input operator resolves to a compiled kernel
    for op in ("softmax_bwd", "layernorm_bwd"):
        for plan in C.credit_enumerate_plans(op, "f32", 2048, 65536):
            assert C.lib().credit_run_plan(C.OPS[op], None, 1, 1, 0.0, 0, ctypes.byref(plan), None) == 1


def test_calibration_loader(tmp_path):
    L = C.lib()
    assert L.credit_load_calibration(str(tmp_path / "missing.json").encode()) == 6
    bad = tmp_path / "bad.json"
    bad.write_text("{ not json")
    assert L.credit_load_calibration(str(bad).encode()) == 6
    noversion = tmp_path / "nov.json"
    noversion.write_text(json.dumps({"stream_gbs": 5000}))
    assert L.credit_load_calibration(str(noversion).encode()) == 6
    invalid = tmp_path / "invalid.json"
    invalid.write_text(json.dumps({"version": 1, "model": {"bw_gbs": 0.0}}))
    assert L.credit_load_calibration(str(invalid).encode()) == 6
    good = tmp_path / "good.json"
    good.write_text(json.dumps({"version": 1, "model": {"bw_gbs": 1000.0, "launch_us": 2.0},
                                "device": {"cus": 256, "xcds": 8}}))
    assert L.credit_load_calibration(str(good).encode()) == 0
    slow = C.credit_select_path("softmax", "f32", 4096, 4096).predicted_us[0]
    assert L.credit_load_calibration(None) == 0
    fast = C.credit_select_path("softmax", "f32", 4096, 4096).predicted_us[0]
    assert slow > fast  # 1000 GB/s model streaming is slower than the default model


def test_make_plan_matches_selector_and_honours_forced_paths():
    for op, dt, rows, cols in [("softmax", "f32", 64, 4096), ("layernorm", "bf16", 4096, 8192),
                               ("rmsnorm", "bf16", 1024, 65536), ("softmax", "f32", 256, 262144)]:
        a = C.credit_select_path(op, dt, rows, cols).as_dict()
        b = C.credit_plan(op, dt, rows, cols).as_dict()
        assert a == b
    p = C.credit_plan("softmax", "f32", 256, 262144, "split", 8)
    assert p.path == C.PATH_SPLIT_ROW and p.split_p == 8
    p = C.credit_plan("layernorm", "bf16", 4096, 8192, "reread")
    assert p.path == C.PATH_REREAD and p.split_p == 1
    with pytest.raises(C.CreditError) as ei:
        C.credit_plan("softmax", "f32", 256, 262144, "single")
    assert ei.value.status == 4
    assert C.lib().credit_make_plan(0, 0, 4, 64, 2, 3, ctypes.byref(C.Plan())) == 1
    assert C.lib().credit_make_plan(0, 0, 4, 64, 0, 0, None) == 1


def test_bf16_layernorm_backward_plans():
    # bf16 LayerNorm backward holds rows of whole 64-byte lines as such and,
    # on the single path, its other rows from the line below their start;
    # its split slices of rows that end in a partial vector are held by
    # element (one-element split tiles)
    C.credit_load_calibration(None)
    try:
        p = C.credit_plan("layernorm_bwd", "bf16", 64, 8192, "single")
        assert p.vec_bytes == 16 and p.block_threads * p.items * 8 >= 8192
        assert 2 * p.items * 16 <= 256 or p.block_threads < 512
        assert C.credit_plan("layernorm_bwd", "bf16", 64, 1002, "single").vec_bytes == 16
        assert C.credit_plan("layernorm_bwd", "bf16", 64, 1002, "reread").vec_bytes == 2
        assert C.credit_plan("layernorm_bwd", "f32", 64, 1001, "single").vec_bytes == 16
    finally:
        C.credit_load_calibration(C.CALIB_PATH if os.path.exists(C.CALIB_PATH) else None)
