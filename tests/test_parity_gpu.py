"""Parity of the HIP path (through the C ABI) with the oracle.

Every case generates seeded inputs on the host, runs the oracle on the CPU and
the library on the GPU, and compares element by element under the tolerances
in tests/parity.py.  Cases: every path (and every split width P) on the named
workloads at full size (the three further workloads compared on a sample of
rows); small shapes that span several tiles with ragged tails for every tile of
every ladder of every operator; one-element-access rows (byte length not a
multiple of 16); and the degenerate shapes (one row, one column, rows = 0, in
place, rows below the CU count, many split rows).
"""
import zlib

import numpy as np
import pytest

from wide_reduction_reuse_amd import workloads as W

from parity import check_result, compare, from_device, oracle_output, to_device

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


def _device_operands(inp):
    w = inp.workload
    return W.alloc_outputs(w, {k: to_device(getattr(inp, k), w.dtype) for k in ("x", "dy", "gamma", "beta")})


def _run(inp, path="auto", split_p=0, plan=None, t=None):
    """Run inp's operator; returns host copies {"y": ..., "row_out": ...}.
    `t`: a prepared operand mapping (e.g. with y aliasing an input)."""
    import torch
    C = _lib()
    w = inp.workload
    t = _device_operands(inp) if t is None else t
    if plan is not None:
        C.credit_run_plan(w.op, plan, t, eps=inp.eps)
    else:
        C.run(w.op, t, inp.eps, path=path, split_p=split_p)
    torch.cuda.synchronize()
    C.credit_check_errors()
    return {"y": from_device(t["y"], w.dtype),
            "row_out": None if t.get("row_out") is None else t["row_out"].cpu().numpy()}


def _check(inp, out, label, rows=None):
    v = check_result(inp, out, rows)
    print("%s: %s" % (label, v), flush=True)
    assert v.ok, "%s: %s" % (label, v)
    return v


def _same(a, b):
    return np.array_equal(a["y"], b["y"]) and (a["row_out"] is None or np.array_equal(a["row_out"], b["row_out"]))


# ---------------------------------------------------------------------------
# named workloads at full size, every legal path
# ---------------------------------------------------------------------------
# rows too wide for one owner of the operator's path-1 tiles (two inputs hold
# twice the bytes): path 1 is refused for these
NO_SINGLE = {"softmax_f32_256x262144", "softmax_bwd_f32_4096x65536", "layernorm_bwd_f32_2048x65536"}
NAMED_CASES = []
for name in W.CONFIG_ORDER + W.NEXT_ORDER + W.EXTRA_ORDER:
    NAMED_CASES.append((name, "auto", 0))
    NAMED_CASES.append((name, "reread", 0))
    for p in (2, 4, 8):
        NAMED_CASES.append((name, "split", p))
    NAMED_CASES.append((name, "single", 0))

_INPUTS = {}


def _named_inputs(name):
    # the generated inputs of the last named workload, reused across its paths
    if name not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[name] = W.generate(W.NAMED[name])
    return _INPUTS[name]


@pytest.mark.parametrize("name,path,p", NAMED_CASES, ids=["%s-%s%s" % (n, pa, p or "") for n, pa, p in NAMED_CASES])
def test_named_workload(name, path, p):
    C = _lib()
    inp = _named_inputs(name)
    try:
        out = _run(inp, path, p)
    except C.CreditError as e:
        # a split too narrow for P, or a row too wide for path 1, is refused
        # before launch, never run
        assert e.status == 4 and (path == "split" or (path == "single" and name in NO_SINGLE)), str(e)
        pytest.skip("%s P=%d cannot hold this row" % (path, p))
    assert not (path == "single" and name in NO_SINGLE)
    rows = None
    if name in W.NEXT_ORDER:
        # the oracle on a sample of rows spread over the whole output
        rows = np.unique(np.concatenate([np.arange(0, inp.workload.rows, 61), [inp.workload.rows - 1]]))
        out = {k: (None if v is None else v[rows]) for k, v in out.items()}
    _check(inp, out, "%s %s P=%d" % (name, path, p), rows)


@pytest.mark.parametrize("op,dt,rows,cols", [("softmax", "f32", 9000, 131072),
                                             ("rmsnorm", "bf16", 17000, 131072)])
def test_tensors_beyond_4_gib(op, dt, rows, cols):
    # 4.4 GiB inputs and outputs (the bf16 one holds more than 2^31
    # elements): row and slice offsets past every 32-bit limit, on the
    # selected plan; the oracle on rows spread over the whole tensor, the
    # last one included
    import torch
    w = W.custom(op, dt, rows, cols, seed=91)
    assert w.rows * w.cols * (4 if dt == "f32" else 2) > (4 << 30)
    inp = W.generate(w)
    out = _run(inp)
    sample = np.unique(np.concatenate([np.arange(0, rows, 997), [rows // 2, rows - 2, rows - 1]]))
    out = {k: (None if v is None else v[sample]) for k, v in out.items()}
    _check(inp, out, "beyond 4 GiB %s %s %dx%d" % (op, dt, rows, cols), sample)
    torch.cuda.empty_cache()


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


# operators whose held tiles hold rows that are not whole 64-byte lines from
# the line boundary below each row's start (RMSNorm's parameter vector, and
# LayerNorm's two, realigned to each row; LayerNorm shifts its odd-length
# bf16 rows only, and holds its other rows as they are or with a partial
# last vector)
SHIFT_OPS = ("softmax", "softmax_bwd", "quantize_int8", "rmsnorm", "layernorm", "layernorm_bwd")
# (LayerNorm's fp32 rows are not shifted, nor are LayerNorm backward's on the
# split path: the tests below hold them as the library does)
SHIFT_CASES = [(op, dt) for op in SHIFT_OPS for dt in W.DTYPES]


def _split_may_not_hold(op, dt):
    """bf16 LayerNorm backward's split slices of rows that are not whole
    16-byte vectors use one-element tiles, of which few are compiled."""
    return op == "layernorm_bwd" and dt == "bf16"


def _row_kind(op, dt, cols, path="single"):
    """The library's row kind (held_row_kind) on the held path, restated: 2
    shifted, 1 a partial last vector, 0 whole vectors (or one-element tiles).
    LayerNorm backward shifts on the single path only: fp32 rows of whole
    16-byte vectors, bf16 rows that are not."""
    nbytes = cols * W.ELEM_BYTES[dt]
    if op == "layernorm_bwd":
        if dt == "f32" and nbytes % 16:
            return 1
        v16 = nbytes % 16 == 0
        return 2 if path == "single" and nbytes % 64 and v16 == (dt == "f32") else 0
    if op in ("softmax", "softmax_bwd", "quantize_int8", "rmsnorm") or (op == "layernorm" and nbytes % 4):
        return 2 if nbytes % 64 else 0
    if op == "layernorm":
        return 1 if nbytes % 16 and nbytes % 4 == 0 else 0
    return 0


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
            if (op, dt) not in W.SUPPORTED:
                continue
            epv = 16 // W.ELEM_BYTES[dt]
            for kind, tiles in ladders.items():
                for block, items in tiles:
                    cap = block * items  # vectors
                    # the operators without parameters hold rows that are not
                    # whole 64-byte lines shifted (test_every_tile_shifted):
                    # here their rows are whole lines (vector counts a
                    # multiple of 4), held as they are
                    lines = op in SHIFT_OPS
                    if kind == "split":
                        for p in (2, 4, 8):
                            # slices fill most of the tile, last slice ragged
                            nv = p * cap - 4 * p - 4 if lines else p * cap - 3 * p - 1
                            cases.append((op, dt, kind, block, items, p, nv * epv))
                    elif kind == "reread":
                        cases.append((op, dt, kind, block, items, 1, (3 * cap + 5) * epv))
                    else:
                        cases.append((op, dt, kind, block, items, 1, (cap - (4 if lines else 3)) * epv))
    return cases


TILE_CASES = _tile_cases()


def _tile_excluded(op, kind, block, items, vb=16, dt="f32", shift=False):
    """The tiles the kernel registry leaves out (they spilled registers): its
    rule restated, so that the library's refusals are checked against it."""
    if shift and op == "layernorm" and kind == "wg" and block == 1024 and items == 16:
        return True
    if op == "layernorm_bwd" and dt == "bf16" and kind != "reread" and block >= 512 and 2 * items * vb > 256:
        return True
    if kind == "reread" or block < 1024:
        return False
    held = W.N_INPUTS.get(op, 1) * items * max(vb, 4)  # a 2-byte vector takes a 32-bit register
    if op == "layernorm" and kind == "split" and items == 16 and vb == 16:
        return True
    if op == "softmax_bwd" and held > (128 if kind == "split" else 256):
        return True
    return op == "layernorm_bwd" and held > 64


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
    if _tile_excluded(op, kind, block, items, dt=dt):
        with pytest.raises(C.CreditError) as ei:
            _run(inp, plan=plan)
        assert ei.value.status == 2  # CREDIT_ERR_UNSUPPORTED, refused before launch
        return
    out = _run(inp, plan=plan)
    _check(inp, out, "tile %s %dx%d p=%d %s %s cols=%d" % (kind, block, items, p, op, dt, cols))


# ---------------------------------------------------------------------------
# rows whose last 16-byte vector is partial: the held tiles of LayerNorm and
# fp32 LayerNorm backward (whose parameters enter the reduction) hold such
# rows as 16-byte vectors from their first byte and mask the missing elements
# of the last one
# ---------------------------------------------------------------------------
PART_OPS = ("layernorm", "layernorm_bwd")


def _partial_tile_cases():
    cases = []
    ladders = {"wave": _ladder("CREDIT_WAVE_TILES"), "wg": _ladder("CREDIT_WG_TILES"),
               "split": _ladder("CREDIT_SPLIT_TILES")}
    i = 0
    for op in PART_OPS:
        for dt in W.DTYPES:
            # bf16 LayerNorm backward reduces its held rows in the streaming
            # form and keeps one-element tiles for such rows
            if (op, dt) not in W.SUPPORTED or (op, dt) == ("layernorm_bwd", "bf16"):
                continue
            epv = 16 // W.ELEM_BYTES[dt]
            tails = (1, 2, 3) if dt == "f32" else (2, 4, 6)  # elements in the partial vector
            for kind, tiles in ladders.items():
                for block, items in tiles:
                    cap = block * items
                    for fill in ("ragged", "full"):
                        ntail = tails[i % 3]
                        i += 1
                        if kind == "split":
                            for p in (2, 4, 8):
                                nv = p * cap - 3 * p - 1 if fill == "ragged" else p * cap
                                cases.append((op, dt, kind, block, items, p, (nv - 1) * epv + ntail))
                        else:
                            nv = cap - 3 if fill == "ragged" else cap
                            cases.append((op, dt, kind, block, items, 1, (nv - 1) * epv + ntail))
    return cases


PARTIAL_TILE_CASES = _partial_tile_cases()


@pytest.mark.parametrize("op,dt,kind,block,items,p,cols", PARTIAL_TILE_CASES,
                         ids=["%s-%s-%s%dx%d-p%d-c%d" % c for c in PARTIAL_TILE_CASES])
def test_every_tile_partial_last_vector(op, dt, kind, block, items, p, cols):
    # The partial vector sits at a different thread and item in each case
    # (the row 3 vectors short of the tile, or filling it); owners loop over
    # rows as in test_every_tile.
    C = _lib()
    rows = {"wave": 1100, "wg": 300, "split": 300}[kind]
    if cols * rows > 24_000_000:
        rows = max(5, 24_000_000 // cols)
    w = W.custom(op, dt, rows, cols, seed=zlib.crc32(("part%s%s%s%d%d%d%d" % (op, dt, kind, block, items, p, cols)).encode()) % 10000,
                 x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    path = C.PATH_SPLIT_ROW if kind == "split" else C.PATH_SINGLE_WG
    plan = C.Plan.make(path, p, block, items, 16, wgs_per_cu=1)
    if _tile_excluded(op, kind, block, items, dt=dt):
        with pytest.raises(C.CreditError) as ei:
            _run(inp, plan=plan)
        assert ei.value.status == 2
        return
    out = _run(inp, plan=plan)
    _check(inp, out, "partial tile %s %dx%d p=%d %s %s cols=%d" % (kind, block, items, p, op, dt, cols))


# ---------------------------------------------------------------------------
# rows that are not whole 64-byte lines, of the operators with shifted rows:
# their held tiles hold each row from the 64-byte boundary below its start,
# with up to 64 - min(g, 16) bytes of the previous row in front (g the lowest
# set bit of the row's byte length), masked and never written; the vectors at
# the row's ends are written byte by byte where they are shared
# ---------------------------------------------------------------------------
def _shift_held_vectors(op, cols, eb, path="single"):
    """The 16-byte vectors the held span of a row needs on `path` (the
    library's rule, restated): shifted rows are held from the 64-byte line
    below their start, with up to 64 - min(g, 16) bytes in front (g the
    lowest set bit of the byte length); other rows as they are."""
    nbytes = cols * eb
    if _row_kind(op, "f32" if eb == 4 else "bf16", cols, path) != 2:
        return (nbytes + 15) // 16
    g = nbytes & -nbytes
    return (nbytes + 64 - min(g, 16) + 15) // 16


def _slice_vectors(nv, p):
    """16-byte vectors per slice (the library's rule, restated): ceil(nv / p)
    rounded up to whole 64-byte lines."""
    return ((nv + p - 1) // p + 3) // 4 * 4


def _shift_cols(op, eb, cls, fits):
    """The widest row of byte-length class `cls` ("odd": odd bf16 length,
    "part": a multiple of 4 bytes but not of 16, "v16": of 16 but not of 64)
    whose held vectors satisfy fits(n)."""
    cols = 1
    while fits(_shift_held_vectors(op, cols, eb)):
        cols *= 2
    while cols > 0:
        nbytes = cols * eb
        ok = {"odd": nbytes % 4 == 2, "part": nbytes % 4 == 0 and nbytes % 16 != 0,
              "v16": nbytes % 16 == 0 and nbytes % 64 != 0}[cls]
        if ok and fits(_shift_held_vectors(op, cols, eb)):
            return cols
        cols -= 1
    return None


def _shift_tile_cases():
    cases = []
    ladders = {"wave": _ladder("CREDIT_WAVE_TILES"), "wg": _ladder("CREDIT_WG_TILES"),
               "split": _ladder("CREDIT_SPLIT_TILES")}
    i = 0
    for op, dt in SHIFT_CASES:
        eb = W.ELEM_BYTES[dt]
        if op == "layernorm":  # shifts its odd-length bf16 rows only
            classes = ("odd",) if dt == "bf16" else ()
        elif op == "layernorm_bwd":  # fp32: rows of whole 16-byte vectors; bf16: the others
            classes = ("odd", "part") if dt == "bf16" else ("v16",)
        else:
            classes = ("odd", "part", "v16") if dt == "bf16" else ("part", "v16")
        if not classes:
            continue
        for kind, tiles in ladders.items():
            if kind == "split" and op == "layernorm_bwd":
                continue  # its split slices are not shifted
            for block, items in tiles:
                cap = block * items
                for fill in ("ragged", "full"):
                    cls = classes[i % len(classes)]
                    i += 1
                    if kind == "split":
                        for p in (2, 4, 8):
                            if fill == "full":  # the widest slice fills the tile
                                fits = lambda n, p=p: (n + p - 1) // p <= cap
                            else:
                                fits = lambda n, p=p: n <= p * cap - 3 * p - 1
                            cases.append((op, dt, kind, block, items, p, _shift_cols(op, eb, cls, fits)))
                    else:
                        lim = cap if fill == "full" else cap - 3
                        cases.append((op, dt, kind, block, items, 1,
                                      _shift_cols(op, eb, cls, lambda n: n <= lim)))
    return cases


SHIFT_TILE_CASES = _shift_tile_cases()


@pytest.mark.parametrize("op,dt,kind,block,items,p,cols", SHIFT_TILE_CASES,
                         ids=["%s-%s-%s%dx%d-p%d-c%d" % c for c in SHIFT_TILE_CASES])
def test_every_tile_shifted(op, dt, kind, block, items, p, cols):
    # An odd row count and owners looping over rows as in test_every_tile: the
    # rows start at every offset their byte length allows inside a 64-byte
    # line, so the row's first and last elements sit at a different thread,
    # item and byte in each row; "full" cases need every held vector of the
    # tile (or slice) for the rows with the largest offset.
    C = _lib()
    rows = {"wave": 1101, "wg": 301, "split": 301}[kind]
    if cols * rows > 24_000_000:
        rows = max(5, 24_000_000 // cols) | 1
    w = W.custom(op, dt, rows, cols,
                 seed=zlib.crc32(("shift%s%s%s%d%d%d%d" % (op, dt, kind, block, items, p, cols)).encode()) % 10000,
                 x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    path = C.PATH_SPLIT_ROW if kind == "split" else C.PATH_SINGLE_WG
    plan = C.Plan.make(path, p, block, items, 16, wgs_per_cu=1)
    if _tile_excluded(op, kind, block, items, dt=dt, shift=_row_kind(op, dt, cols) == 2):
        with pytest.raises(C.CreditError) as ei:
            _run(inp, plan=plan)
        assert ei.value.status == 2
        return
    out = _run(inp, plan=plan)
    _check(inp, out, "shifted tile %s %dx%d p=%d %s %s cols=%d" % (kind, block, items, p, op, dt, cols))


@pytest.mark.parametrize("op,dt", SHIFT_CASES)
def test_shifted_tile_one_vector_short_is_refused(op, dt):
    # a tile that holds the row but not the row with its largest offset in
    # front is refused before launch
    C = _lib()
    eb = W.ELEM_BYTES[dt]
    cols = _shift_cols(op, eb, ("v16" if op == "layernorm_bwd" else "part") if dt == "f32" else "odd",
                       lambda n: n <= 257)
    assert _shift_held_vectors(op, cols, eb) == 257
    w = W.custom(op, dt, 3, cols, seed=3)
    inp = W.generate(w)
    with pytest.raises(C.CreditError) as ei:
        _run(inp, plan=C.Plan.make(C.PATH_SINGLE_WG, 1, 64, 4, 16))
    assert ei.value.status == 4


@pytest.mark.parametrize("cols", [1, 5, 100, 1001, 1004, 30001])
@pytest.mark.parametrize("xoff,yoff", [(16, 0), (48, 32), (0, 16)])
@pytest.mark.parametrize("op,dt", SHIFT_CASES)
def test_shifted_rows_with_offset_bases(op, dt, xoff, yoff, cols):
    # x (and dy) and y start 0-48 bytes into a 64-byte line, differently: the
    # offset of each row is taken from x's address, the first rows (less than
    # 64 bytes into x) are held from the tensor's start, and y's held spans
    # are then 16-byte but not line aligned.  Single and split paths.
    import torch
    C = _lib()
    w = W.custom(op, dt, 19, cols, seed=cols + xoff + 3 * yoff, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    for path, p in (("single", 0), ("split", 2)):
        if path == "split" and _split_may_not_hold(op, dt):
            continue
        t = _device_operands(inp)

        def moved(a, off):
            if a is None:
                return None
            nb = a.numel() * a.element_size()
            buf = torch.empty(nb + 128, dtype=torch.uint8, device="cuda")
            base = (-buf.data_ptr()) % 64 + off
            v = buf[base: base + nb].view(a.dtype).view(a.shape)
            v.copy_(a)
            return v

        for k in ("x", "dy"):
            t[k] = moved(t.get(k), xoff)
        t["y"] = moved(t["y"], yoff)
        assert t["x"].data_ptr() % 64 == xoff and t["y"].data_ptr() % 64 == yoff
        nvh = _shift_held_vectors(op, cols, W.ELEM_BYTES[dt], path)
        if path == "split" and nvh <= _slice_vectors(nvh, 2):
            continue  # too narrow to split
        out = _run(inp, path, p, t=t)
        _check(inp, out, "offset bases x+%d y+%d %s %s cols=%d %s" % (xoff, yoff, op, dt, cols, path))


@pytest.mark.parametrize("dt,cols", [("bf16", 1), ("bf16", 7), ("bf16", 12291), ("f32", 3), ("f32", 1004),
                                     ("f32", 12291)])
@pytest.mark.parametrize("path,p", [("single", 0), ("split", 2), ("split", 8), ("reread", 0)])
@pytest.mark.parametrize("op,alias", [("softmax", "x"), ("softmax_bwd", "x"), ("softmax_bwd", "dy"),
                                      ("layernorm_bwd", "x"), ("layernorm_bwd", "dy")])
def test_shifted_rows_in_place_and_boundary_nan(op, alias, dt, path, p, cols):
    # The output overwrites an input while the neighbouring rows' owners read
    # the 64-byte lines they share with this row; then NaN in the first and
    # last elements of some rows (x, and dy for the backward operator) must
    # stay in those rows.
    if path == "split" and _split_may_not_hold(op, dt):
        pytest.skip("%s %s split slices are not shifted" % (op, dt))
    C = _lib()
    eb = W.ELEM_BYTES[dt]
    nvh = _shift_held_vectors(op, cols, eb, path)
    if path == "split" and nvh <= (p - 1) * _slice_vectors(nvh, p):
        pytest.skip("too narrow to split %d ways" % p)
    w = W.custom(op, dt, 37, cols, seed=cols + 3, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    t = _device_operands(inp)
    t["y"] = t[alias]
    out = _run(inp, path, p, t=t)
    _check(inp, out, "shifted in-place y=%s %s %s %s P=%d cols=%d" % (alias, op, dt, path, p, cols))
    nan = np.uint16(0x7FC0) if dt == "bf16" else np.float32("nan")
    bad = (5, 6, 20)
    inp.x[5, 0] = nan
    inp.x[6, cols - 1] = nan
    if inp.dy is not None:
        inp.dy[20, 0] = nan
        inp.dy[20, cols - 1] = nan
    else:
        inp.x[20, cols - 1] = nan
    y = _run(inp, path, p)["y"]
    isnan = np.isnan((y.astype(np.uint32) << 16).view(np.float32)) if dt == "bf16" else np.isnan(y)
    for r in range(w.rows):
        if r in bad:
            assert isnan[r].all(), "row %d should be NaN" % r
        else:
            assert not isnan[r].any(), "NaN leaked into row %d" % r


@pytest.mark.parametrize("op,path,p", [(op, path, p) for op in SHIFT_OPS for path, p in (("single", 0), ("split", 4))
                                         if op != "layernorm_bwd" or path == "single"])
def test_odd_length_bf16_word_after_the_tensor_is_masked(op, path, p):
    # rows * cols odd: the last row ends in the middle of a 4-byte word whose
    # other half lies after the tensor; the kernels read that word and must
    # mask it.  Here it holds a NaN (x and dy are views of longer buffers).
    import torch
    C = _lib()
    rows, cols = 35, 4099
    w = W.custom(op, "bf16", rows, cols, seed=17)
    inp = W.generate(w)
    t = _device_operands(inp)
    for k in ("x", "dy"):
        if t.get(k) is None:
            continue
        buf = torch.empty(rows * cols + 8, dtype=torch.bfloat16, device="cuda")
        buf.view(torch.int16)[rows * cols:] = 0x7FC0  # NaN after the tensor
        buf[: rows * cols].copy_(t[k].reshape(-1))
        t[k] = buf[: rows * cols].view(rows, cols)
    out = _run(inp, path, p, t=t)
    _check(inp, out, "word after the tensor %s %s P=%d" % (op, path, p))


# ---------------------------------------------------------------------------
# rows whose byte length is not a multiple of 16: partial last vectors
# (above) and one-element accesses (odd bf16 lengths, int8 quantization,
# LayerNorm backward, the reread path)
# ---------------------------------------------------------------------------
ODD_CASES = [(op, dt, cols, path, p)
             for op in W.OPS for dt in W.DTYPES if (op, dt) in W.SUPPORTED
             for cols, path, p in [(1, "auto", 0), (2, "auto", 0), (3, "auto", 0), (6, "auto", 0),
                                   (1001, "auto", 0), (1001, "reread", 0), (1002, "auto", 0),
                                   (16382, "single", 0), (16383, "single", 0), (30001, "split", 2),
                                   (30001, "reread", 0), (30002, "split", 2), (60007, "split", 4),
                                   (50257, "auto", 0), (100003, "auto", 0), (100003, "split", 8),
                                   (100006, "split", 8)]]


@pytest.mark.parametrize("op,dt,cols,path,p", ODD_CASES, ids=["%s-%s-c%d-%s%d" % c for c in ODD_CASES])
def test_unaligned_row_lengths(op, dt, cols, path, p):
    C = _lib()
    w = W.custom(op, dt, 6, cols, seed=cols + 7, x_dist="scaled_shifted", x_scale=2.0, x_shift=-0.25)
    inp = W.generate(w)
    if (op, dt) == ("layernorm_bwd", "bf16") and path == "split" and cols * 2 % 16 != 0:
        # its split slices of such rows would be held by element, and its
        # one-element tiles end at 1024 x 4 (larger ones spilled registers;
        # on the single path such rows are shifted): a forced split is
        # refused before launch
        with pytest.raises(C.CreditError) as ei:
            _run(inp, path, p)
        assert ei.value.status == 4
        return
    out = _run(inp, path, p)
    _check(inp, out, "odd %s %s cols=%d %s P=%d" % (op, dt, cols, path, p))


# ---------------------------------------------------------------------------
# degenerate and structural cases
# ---------------------------------------------------------------------------
SUPPORTED_CASES = sorted(W.SUPPORTED)


@pytest.mark.parametrize("op,dt", SUPPORTED_CASES)
def test_single_column(op, dt):
    inp = W.generate(W.custom(op, dt, 37, 1, seed=11))
    out = _run(inp)
    _check(inp, out, "cols=1 %s %s" % (op, dt))


@pytest.mark.parametrize("path,p", [("single", 0), ("split", 4), ("reread", 0)])
def test_rows_zero_is_noop(path, p):
    import torch
    C = _lib()
    x = torch.empty((0, 4096), device="cuda")
    y = torch.full((0, 4096), 7.0, device="cuda")
    C.credit_softmax(x, y, path, p)
    torch.cuda.synchronize()
    assert y.numel() == 0


IN_PLACE_CASES = [(op, alias) for op in W.OPS if op != "quantize_int8"
                  for alias in (("x", "dy") if W.N_INPUTS.get(op, 1) == 2 else ("x",))]


@pytest.mark.parametrize("cols", [12288, 12290])
@pytest.mark.parametrize("path,p", [("single", 0), ("split", 2), ("split", 8), ("reread", 0)])
@pytest.mark.parametrize("op,alias", IN_PLACE_CASES)
def test_in_place(op, alias, path, p, cols):
    # the output overwrites an input (the int8 quantizer's output has another
    # type); 12290 columns end in a partial vector
    C = _lib()
    w = W.custom(op, "f32", 33, cols, seed=5, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    t = _device_operands(inp)
    t["y"] = t[alias]
    out = _run(inp, path, p, t=t)
    _check(inp, out, "in-place y=%s %s %s P=%d cols=%d" % (alias, op, path, p, cols))


@pytest.mark.parametrize("op", W.OPS)
def test_split_bitwise_deterministic_and_many_rows(op):
    # 50000 rows exceed one launch's exchange capacity for P=8 (several launches)
    dt = "bf16" if (op, "bf16") in W.SUPPORTED else "f32"
    w = W.custom(op, dt, 50000, 256, seed=21, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    y1 = _run(inp, "split", 8)
    y2 = _run(inp, "split", 8)
    assert _same(y1, y2)
    _check(inp, y1, "many rows split P=8 %s" % op)


@pytest.mark.parametrize("op,dt", SUPPORTED_CASES)
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
    assert _same(ys[0], ys[1]) and _same(ys[0], ys[2])


@pytest.mark.parametrize("cols", [32768, 32764])
@pytest.mark.parametrize("op,dt", SUPPORTED_CASES)
def test_paths_agree_closely(op, dt, cols):
    # all legal paths on one shape: each within tolerance of the oracle, and
    # path 1 bitwise stable run to run (32764 columns end in a partial vector)
    C = _lib()
    w = W.custom(op, dt, 40, cols, seed=31)
    inp = W.generate(w)
    ys = {}
    for path, p in [("single", 0), ("split", 2), ("split", 4), ("split", 8), ("reread", 0)]:
        if (op, dt) == ("layernorm_bwd", "bf16") and cols % 8 != 0 and path != "reread":
            # rows ending in a partial vector: one-element tiles up to 4096
            # elements only (see test_unaligned_row_lengths)
            with pytest.raises(C.CreditError) as ei:
                _run(inp, path, p)
            assert ei.value.status == 4
            continue
        ys[(path, p)] = _run(inp, path, p)
        _check(inp, ys[(path, p)], "agree %s %s %s P=%d" % (op, dt, path, p))
    if ("single", 0) in ys:
        assert _same(ys[("single", 0)], _run(inp, "single", 0))


def test_rows_fewer_than_cus_and_odd_row_counts():
    for rows in (1, 3, 255, 257):
        inp = W.generate(W.custom("layernorm", "bf16", rows, 8192, seed=rows))
        for path, p in [("single", 0), ("split", 4), ("reread", 0)]:
            _check(inp, _run(inp, path, p), "rows=%d %s" % (rows, path))
    for rows in (1, 255):
        inp = W.generate(W.custom("quantize_int8", "f32", rows, 8192, seed=rows, x_dist="outliers",
                                  outlier_prob=0.01, outlier_scale=50.0))
        for path, p in [("single", 0), ("split", 4), ("reread", 0)]:
            _check(inp, _run(inp, path, p), "quantize rows=%d %s" % (rows, path))


@pytest.mark.parametrize("cols", [32768, 32766])
@pytest.mark.parametrize("op", ["softmax", "softmax_bwd"])
def test_masked_runs_of_logits(op, cols):
    # Rows with long runs of very negative logits, as from a mask: whole
    # groups of a thread's vectors whose own maximum lies ~1e4 below the
    # row's, so the factor that rescales them to the row maximum underflows
    # to zero; and rows with a single unmasked element (a one-hot output).
    # 32766 columns end in a partial vector.
    w = W.custom(op, "f32", 64, cols, seed=77, x_dist="scaled_shifted", x_scale=2.0, x_shift=0.0)
    inp = W.generate(w)
    rng = np.random.default_rng(77)
    cols = w.cols
    for r in range(w.rows):
        kind = r % 4
        if kind == 0:
            inp.x[r, : cols // 2] -= 1e4
        elif kind == 1:
            inp.x[r, cols // 2 :] -= 1e4
        elif kind == 2:
            for c0 in range(0, cols, 1024):
                inp.x[r, c0 : c0 + 512] -= 1e4
        else:
            keep = int(rng.integers(0, cols))
            inp.x[r, :] -= 1e4
            inp.x[r, keep] = 0.0
    for path, p in [("auto", 0), ("single", 0), ("split", 2), ("split", 4), ("split", 8), ("reread", 0)]:
        if path == "single" and op == "softmax_bwd" and _shift_held_vectors(op, cols, 4) > 8192:
            # a shifted 32766-column row spans 8195 vectors, more than softmax
            # backward's largest path-1 tile (1024 x 8) holds: refused
            with pytest.raises(C.CreditError) as ei:
                _run(inp, path, p)
            assert ei.value.status == 4
            continue
        _check(inp, _run(inp, path, p), "masked %s %s P=%d cols=%d" % (op, path, p, cols))


@pytest.mark.parametrize("cols", [8192, 8190, 8191])
@pytest.mark.parametrize("op,dt", [("softmax", "f32"), ("softmax", "bf16"), ("softmax_bwd", "f32"),
                                   ("softmax_bwd", "bf16")])
def test_logits_masked_to_the_lowest_finite_value(op, dt, cols):
    # A masked fill with the dtype's lowest finite value (float32 -3.4028e38,
    # bf16 -3.3895e38): x - max lies below -FLT_MAX / log2 e, where the product
    # x log2 e overflows; such entries must come out 0.  Rows half masked,
    # all but ~1% masked, and fully masked (a uniform softmax).  8190 columns
    # end in a partial vector; 8191 bf16 columns are an odd-length row.
    w = W.custom(op, dt, 48, cols, seed=78)
    inp = W.generate(w)
    rng = np.random.default_rng(78)
    fill = np.float32(np.finfo(np.float32).min) if dt == "f32" else np.uint16(0xFF7F)
    for r in range(w.rows):
        kind = r % 3
        mask = rng.random(w.cols) < (0.5 if kind == 0 else 0.99)
        if kind == 2:
            mask[:] = True
        inp.x[r, mask] = fill
    for path, p in [("auto", 0), ("single", 0), ("split", 2), ("split", 4), ("reread", 0)]:
        _check(inp, _run(inp, path, p), "lowest-fill %s %s %s P=%d cols=%d" % (op, dt, path, p, cols))


def test_nan_propagates_to_its_row_only():
    C = _lib()
    inp = W.generate(W.custom("softmax", "f32", 4, 4096, seed=9))
    inp.x[2, 100] = np.nan
    for path, p in [("single", 0), ("split", 4), ("reread", 0)]:
        y = _run(inp, path, p)["y"]
        assert np.all(np.isnan(y[2]))
        yhat = oracle_output(inp, cache=False)
        v = compare("softmax", "f32", np.delete(y, 2, axis=0), np.delete(yhat, 2, axis=0))
        assert v.ok, str(v)
