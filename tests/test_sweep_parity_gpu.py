"""Parity of the 90-point crossover sweep (softmax, LayerNorm and RMSNorm in
fp32 and bf16, widths 1024 ... 262144, 16 MiB, 256 MiB and 1 GiB of input;
the width sweep of the CREDIT paper, Sec. IV-A and IV-B, Fig. 3) with the
oracle, on the plan the selector picks for each shape, through the C ABI.

Inputs are drawn on the device (workloads.device_inputs, seeded per point), so
the 1 GiB shapes need no host-side generation; the rows a check compares are
copied to the host with the parameters and given to the oracle.  Every row is
compared for the 16 MiB points; for the others, 96 rows spread evenly over the
tensor and its last row, so persistent owners that loop over hundreds of rows
are checked at the start, middle and end of their loops.
"""
import numpy as np
import pytest

from wide_reduction_reuse_amd import workloads as W

from parity import check_result, from_device

pytestmark = pytest.mark.gpu

POINTS = W.sweep_points()
FULL_CHECK_BYTES = 16 << 20
SAMPLE_ROWS = 96


def sample_rows(w: W.Workload) -> np.ndarray:
    if w.rows * w.cols * W.ELEM_BYTES[w.dtype] <= FULL_CHECK_BYTES:
        return np.arange(w.rows)
    step = max(1, w.rows // SAMPLE_ROWS)
    return np.unique(np.concatenate([np.arange(0, w.rows, step), [w.rows - 1]]))


@pytest.mark.parametrize("w", POINTS, ids=[w.name for w in POINTS])
def test_sweep_point_on_selected_plan(w):
    import torch
    from wide_reduction_reuse_amd import credit as C
    assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
    t = W.device_inputs(w)
    plan = C.credit_select_path(w.op, w.dtype, w.rows, w.cols)
    C.run(w.op, t, w.eps, path="auto", check=True)
    idx = sample_rows(w)
    sel = torch.from_numpy(idx).to("cuda")
    host = W.HostInputs(w.with_shape(len(idx), w.cols, name=w.name + "_sample"),
                        from_device(t["x"].index_select(0, sel), w.dtype),
                        None if t["gamma"] is None else from_device(t["gamma"], w.dtype),
                        None if t["beta"] is None else from_device(t["beta"], w.dtype),
                        float(np.float32(w.eps)))
    out = {"y": from_device(t["y"].index_select(0, sel), w.dtype), "row_out": None}
    del t
    v = check_result(host, out)
    print("%s plan p%d P=%d %dx%d: %d rows checked, %s" % (w.name, plan.path, plan.split_p, plan.block_threads,
                                                          plan.items, len(idx), v), flush=True)
    assert v.ok, "%s: %s" % (w.name, v)
    torch.cuda.empty_cache()
