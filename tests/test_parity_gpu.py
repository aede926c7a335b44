"""Parity of the HIP path (through the C ABI) with the double-precision oracle.

Every case generates seeded inputs on the host, runs the oracle on the CPU and
the library on the GPU, and compares element by element under the tolerances
in tests/parity.py.  Cases: every path (and every split width P) on the four
named workloads at full size; small shapes that span several tiles with ragged
tails for every tile of every ladder; one-element-access rows (byte length not
a multiple of 16); and the degenerate shapes (one row, one column, rows = 0,
in place, rows below the CU count, many split rows).
"""
import zlib

import numpy as np
import pytest

from wide_reduction_reuse_amd import workloads as W

from parity import compare, from_device, oracle_output, to_device

pytestmark = pytest.mark.gpu

C = None


def _lib():
    global C
    if C is None:
        import torch
        from wide_reduction_reuse_amd import credit
        assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
        C = credit
    return C


def _run(inp, path="auto", split_p=0, plan=None, y=None):
    import torch
    C = _lib()
    w = inp.workload
    x = to_device(inp.x, w.dtype)
    g = to_device(inp.gamma, w.dtype)
    b = to_device(inp.beta, w.dtype)
    if plan is not None:
        out = torch.empty_like(x) if y is None else y
        C.credit_run_plan(w.op, x, g, b, out, inp.eps, plan)
    else:
        out = C.run(w.op, x, g, b, inp.eps, y=y, path=path, split_p=split_p)
    torch.cuda.synchronize()
    C.credit_check_errors()
    return from_device(out, w.dtype)


def _check(inp, y, label):
    v = compare(inp.workload.op, inp.workload.dtype, y, oracle_output(inp))
    print("%s: %s" % (label, v), flush=True)
    assert v.ok, "%s: %s" % (label, v)
    return v


# ---------------------------------------------------------------------------
# named workloads at full size, every legal path
# ---------------------------------------------------------------------------
NAMED_CASES = []
for name in W.CONFIG_ORDER:
    w = W.NAMED[name]
    NAMED_CASES.append((name, "auto", 0))
    NAMED_CASES.append((name, "reread", 0))
    for p in (2, 4, 8):
        NAMED_CASES.append((name, "split", p))
    if not name.startswith("softmax_f32_256x262144"):
        NAMED_CASES.append((name, "single", 0))


@pytest.mark.parametrize("name,path,p", NAMED_CASES, ids=["%s-%s%s" % (n, pa, p or "") for n, pa, p in NAMED_CASES])
def test_named_workload(name, path, p):
    C = _lib()
    inp = W.generate(W.NAMED[name])
    try:
        y = _run(inp, path, p)
    except C.CreditError as e:
        # a split too narrow for P is refused before launch, never run
        assert e.status == 4 and path == "split", str(e)
        pytest.skip("P=%d cannot split this row" % p)
    _check(inp, y, "%s %s P=%d" % (name, path, p))


def test_single_row_too_wide_is_refused():
    C = _lib()
    inp = W.generate(W.NAMED["softmax_f32_256x262144"].with_shape(2, 262144))
    with pytest.raises(C.CreditError) as ei:
        _run(inp, "single")
    assert ei.value.status == 4


# ---------------------------------------------------------------------------
# every compiled tile, on a shape that spans it with a ragged tail
# ---------------------------------------------------------------------------
def _ladder(macro):
    """(block, items) pairs of one X-macro tile list in the kernel registry header."""
    import os
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "wide_reduction_reuse_amd", "csrc", "registry.hpp")).read()
    body = re.search(r"#define %s\(X\)((?:[^\n]*\\\n)*[^\n]*)" % macro, text).group(1)
    pairs = re.findall(r"X\((\d+)(?:,\s*(\d+))?\)", body)
    return [(64, int(a)) if not b else (int(a), int(b)) for a, b in pairs]


def _tile_cases():
    cases = []
    ladders = {
        "wave": _ladder("CREDIT_WAVE_TILES"),
        "wg": _ladder("CREDIT_WG_TILES"),
        "split": _ladder("CREDIT_SPLIT_TILES"),
        "reread": _ladder("CREDIT_REREAD_TILES"),
    }
    for op in W.OPS:
        for dt in W.DTYPES:
            epv = 16 // W.ELEM_BYTES[dt]
            for kind, tiles in ladders.items():
                for block, items in tiles:
                    cap = block * items  # vectors
                    if kind == "split":
                        for p in (2, 4, 8):
                            # slices fill most of the tile, last slice ragged
                            nv = p * cap - 3 * p - 1
                            cases.append((op, dt, kind, block, items, p, nv * epv))
                    elif kind == "reread":
                        cases.append((op, dt, kind, block, items, 1, (3 * cap + 5) * epv))
                    else:
                        cases.append((op, dt, kind, block, items, 1, (cap - 3) * epv))
    return cases


TILE_CASES = _tile_cases()
# tiles the registry leaves out for one operator (they would spill registers)
EXCLUDED_TILES = {("layernorm", "split", 1024, 16)}


@pytest.mark.parametrize("op,dt,kind,block,items,p,cols", TILE_CASES,
                         ids=["%s-%s-%s%dx%d-p%d-c%d" % c for c in TILE_CASES])
def test_every_tile(op, dt, kind, block, items, p, cols):
    # One workgroup per CU (wgs_per_cu = 1) and more rows than owners, so that
    # owners loop over rows (1 to 3 each, ragged) and load each next row while
    # writing the current one; the reread kernel takes one row per workgroup.
    C = _lib()
    rows = {"wave": 1100, "wg": 300, "split": 300, "reread": 5}[kind]
    if cols * rows > 24_000_000:
        rows = max(5, 24_000_000 // cols)
    w = W.custom(op, dt, rows, cols, seed=zlib.crc32(("%s%s%s%d%d%d" % (op, dt, kind, block, items, p)).encode()) % 10000,
                 x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    path = {"wave": C.PATH_SINGLE_WG, "wg": C.PATH_SINGLE_WG, "split": C.PATH_SPLIT_ROW,
            "reread": C.PATH_REREAD}[kind]
    plan = C.Plan.make(path, p, block, items, 16, wgs_per_cu=1)
    if (op, kind, block, items) in EXCLUDED_TILES:
        with pytest.raises(C.CreditError) as ei:
            _run(inp, plan=plan)
        assert ei.value.status == 2  # CREDIT_ERR_UNSUPPORTED, refused before launch
        return
    y = _run(inp, plan=plan)
    _check(inp, y, "tile %s %dx%d p=%d %s %s cols=%d" % (kind, block, items, p, op, dt, cols))


# ---------------------------------------------------------------------------
# rows whose byte length is not a multiple of 16 (one-element accesses)
# ---------------------------------------------------------------------------
ODD_CASES = [(op, dt, cols, path, p)
             for op in W.OPS for dt in W.DTYPES
             for cols, path, p in [(1, "auto", 0), (3, "auto", 0), (1001, "auto", 0), (1001, "reread", 0),
                                   (16383, "single", 0), (30001, "split", 2), (30001, "reread", 0),
                                   (60007, "split", 4)]]


@pytest.mark.parametrize("op,dt,cols,path,p", ODD_CASES, ids=["%s-%s-c%d-%s%d" % c for c in ODD_CASES])
def test_unaligned_row_lengths(op, dt, cols, path, p):
    w = W.custom(op, dt, 6, cols, seed=cols + 7, x_dist="scaled_shifted", x_scale=2.0, x_shift=-0.25)
    inp = W.generate(w)
    y = _run(inp, path, p)
    _check(inp, y, "odd %s %s cols=%d %s P=%d" % (op, dt, cols, path, p))


# ---------------------------------------------------------------------------
# degenerate and structural cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("op", W.OPS)
@pytest.mark.parametrize("dt", W.DTYPES)
def test_single_column(op, dt):
    inp = W.generate(W.custom(op, dt, 37, 1, seed=11))
    y = _run(inp)
    _check(inp, y, "cols=1 %s %s" % (op, dt))


@pytest.mark.parametrize("path,p", [("single", 0), ("split", 4), ("reread", 0)])
def test_rows_zero_is_noop(path, p):
    import torch
    C = _lib()
    x = torch.empty((0, 4096), device="cuda")
    y = torch.full((0, 4096), 7.0, device="cuda")
    C.credit_softmax(x, y, path, p)
    torch.cuda.synchronize()
    assert y.numel() == 0


@pytest.mark.parametrize("path,p", [("single", 0), ("split", 2), ("split", 8), ("reread", 0)])
@pytest.mark.parametrize("op", W.OPS)
def test_in_place(op, path, p):
    import torch
    C = _lib()
    w = W.custom(op, "f32", 33, 12288, seed=5, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    x = to_device(inp.x, "f32")
    g = to_device(inp.gamma, "f32")
    b = to_device(inp.beta, "f32")
    C.run(op, x, g, b, inp.eps, y=x, path=path, split_p=p)
    torch.cuda.synchronize()
    _check(inp, from_device(x, "f32"), "in-place %s %s P=%d" % (op, path, p))


@pytest.mark.parametrize("op", W.OPS)
def test_split_bitwise_deterministic_and_many_rows(op):
    # 50000 rows exceed one launch's exchange capacity for P=8 (several launches)
    C = _lib()
    w = W.custom(op, "bf16", 50000, 256, seed=21, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    y1 = _run(inp, "split", 8)
    y2 = _run(inp, "split", 8)
    assert np.array_equal(y1, y2)
    _check(inp, y1, "many rows split P=8 %s" % op)


@pytest.mark.parametrize("op", W.OPS)
@pytest.mark.parametrize("dt", W.DTYPES)
def test_persistent_owners_match_one_row_per_owner_bitwise(op, dt):
    # the same tile with owners looping over many rows (rolling loads), at full
    # occupancy, and with one row per owner: identical bits, all within tolerance
    C = _lib()
    w = W.custom(op, dt, 5000, 4096, seed=41, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    base = C.credit_plan(op, dt, w.rows, w.cols, "single")
    ys = []
    for wpc in (1, 0, -1):
        plan = C.Plan.make(C.PATH_SINGLE_WG, 1, base.block_threads, base.items, base.vec_bytes, wgs_per_cu=wpc)
        ys.append(_run(inp, plan=plan))
        _check(inp, ys[-1], "persistent %s %s wgs_per_cu=%d" % (op, dt, wpc))
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


@pytest.mark.parametrize("op", W.OPS)
@pytest.mark.parametrize("dt", W.DTYPES)
def test_paths_agree_closely(op, dt):
    # all legal paths on one shape: each within tolerance of the oracle, and
    # path 1 bitwise stable run to run
    w = W.custom(op, dt, 40, 32768, seed=31)
    inp = W.generate(w)
    ys = {}
    for path, p in [("single", 0), ("split", 2), ("split", 4), ("split", 8), ("reread", 0)]:
        ys[(path, p)] = _run(inp, path, p)
        _check(inp, ys[(path, p)], "agree %s %s %s P=%d" % (op, dt, path, p))
    assert np.array_equal(ys[("single", 0)], _run(inp, "single", 0))


def test_rows_fewer_than_cus_and_odd_row_counts():
    for rows in (1, 3, 255, 257):
        inp = W.generate(W.custom("layernorm", "bf16", rows, 8192, seed=rows))
        for path, p in [("single", 0), ("split", 4), ("reread", 0)]:
            _check(inp, _run(inp, path, p), "rows=%d %s" % (rows, path))


def test_nan_propagates_to_its_row_only():
    C = _lib()
    inp = W.generate(W.custom("softmax", "f32", 4, 4096, seed=9))
    inp.x[2, 100] = np.nan
    for path, p in [("single", 0), ("split", 4), ("reread", 0)]:
        y = _run(inp, path, p)
        assert np.all(np.isnan(y[2]))
        yhat = oracle_output(inp, cache=False)
        v = compare("softmax", "f32", np.delete(y, 2, axis=0), np.delete(yhat, 2, axis=0))
        assert v.ok, str(v)
