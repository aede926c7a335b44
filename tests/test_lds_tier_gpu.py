"""Parity of the LDS tier with the oracle, every LDS-tier tile of every
operator and dtype, on paths 1 and 2.

A tile with an LDS part holds block * items vectors of its row (or slice) in
registers and up to block * lds more in LDS.  Each tile is run at two
widths: one vector past its register part (an LDS part of a single vector)
and an LDS part five vectors short of full (its last step partly past the
row); path 1 with workgroups looping over rows (the LDS part refilled for
every row) and with one row per workgroup, path 2 at P = 2 (and P = 4 for
the second width) with clusters looping over rows.  Compared element by
element with the oracle under the tolerances in tests/parity.py.
"""
import re
import os
import zlib

import pytest

from wide_reduction_reuse_amd import workloads as W

from parity import check_result, from_device, to_device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INPUTS = {"softmax_bwd": 2, "layernorm_bwd": 2}


def _lds_ladder(macro):
    """(block, items, lds) triples of an LDS-tier tile list in the kernel registry header."""
    text = open(os.path.join(ROOT, "wide_reduction_reuse_amd", "csrc", "registry.hpp")).read()
    body = re.search(r"#define %s\(X\)([^\n]*)" % macro, text).group(1)
    return [tuple(int(v) for v in t) for t in re.findall(r"X\((\d+),\s*(\d+),\s*(\d+)\)", body)]


def _enabled(op, dt, block, items):
    # the registry's rule: one-input operators but LayerNorm at 1024 threads,
    # every operator at 512 (bf16 LayerNorm backward only with at most 256
    # bytes of x and dy in registers per thread)
    if op == "layernorm_bwd" and dt == "bf16" and 2 * items * 16 > 256:
        return False
    return block < 1024 or (INPUTS.get(op, 1) == 1 and op != "layernorm")


def _cases():
    cases = []
    for kind, macro in (("wg", "CREDIT_WG_LDS_TILES"), ("split", "CREDIT_SPLIT_LDS_TILES")):
        for block, items, lds in _lds_ladder(macro):
            for op in W.OPS:
                for dt in W.DTYPES:
                    if (op, dt) not in W.SUPPORTED or not _enabled(op, dt, block, items):
                        continue
                    reg, cap = block * items, block * (items + lds)
                    for fill, per in (("one", reg + 1), ("ragged", cap - 5)):
                        for p in ((1,) if kind == "wg" else ((2, 4) if fill == "ragged" else (2,))):
                            cases.append((op, dt, kind, block, items, lds, p, fill, per * p))
    return cases


CASES = _cases()


def _lib():
    import torch
    from wide_reduction_reuse_amd import credit
    assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
    return credit


def _run(C, inp, plan):
    import torch
    w = inp.workload
    t = W.alloc_outputs(w, {k: to_device(getattr(inp, k), w.dtype) for k in ("x", "dy", "gamma", "beta")})
    C.credit_run_plan(w.op, plan, t, eps=inp.eps)
    torch.cuda.synchronize()
    C.credit_check_errors()
    return {"y": from_device(t["y"], w.dtype),
            "row_out": None if t.get("row_out") is None else t["row_out"].cpu().numpy()}


@pytest.mark.parametrize("op,dt,kind,block,items,lds,p,fill,nv", CASES,
                         ids=["%s-%s-%s%dx%d+%d-p%d-%s" % c[:8] for c in CASES])
def test_lds_tier_tile(op, dt, kind, block, items, lds, p, fill, nv):
    C = _lib()
    epv = 16 // W.ELEM_BYTES[dt]
    cols = nv * epv
    path = C.PATH_SINGLE_WG if kind == "wg" else C.PATH_SPLIT_ROW
    seed = zlib.crc32(("lds%s%s%s%d%d%d%d%s" % (op, dt, kind, block, items, lds, p, fill)).encode()) % 10000
    # path 1: 260 rows on one workgroup per CU, so that some loop; path 2:
    # more rows than clusters of one workgroup per CU (128 for P = 2, 64 for
    # P = 4) where that stays within 24 M elements
    rows = min(260 if kind == "wg" else (130 if p == 2 else 70), max(8, 24_000_000 // cols))
    w = W.custom(op, dt, rows, cols, seed=seed, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp = W.generate(w)
    plan = C.Plan.make(path, p, block, items, 16, wgs_per_cu=1, lds_items=lds)
    out = _run(C, inp, plan)
    v = check_result(inp, out)
    print("lds tier %s %dx%d+%d p=%d %s %s cols=%d: %s" % (kind, block, items, lds, p, op, dt, cols, v), flush=True)
    assert v.ok, v
    if kind == "wg" and fill == "ragged":
        # one row per workgroup as well
        plan1 = C.Plan.make(path, 1, block, items, 16, wgs_per_cu=-1, lds_items=lds)
        out1 = _run(C, inp, plan1)
        v1 = check_result(inp, out1)
        assert v1.ok, v1


def test_lds_tier_rejects_rows_it_cannot_hold():
    C = _lib()
    # one vector past the LDS part: refused before launch
    w = W.custom("softmax", "f32", 2, 4 * (1024 * 24 + 1), seed=1)
    inp = W.generate(w)
    with pytest.raises(C.CreditError) as e:
        _run(C, inp, C.Plan.make(C.PATH_SINGLE_WG, 1, 1024, 16, 16, wgs_per_cu=-1, lds_items=8))
    assert e.value.status == 4
