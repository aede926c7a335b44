"""The work-free control kernel (the CREDIT paper's control for cluster
overhead, Sec. III-D) on the GPU: for every operator, the control twin of a
split tile at P = 2, 4 and 8 runs with the same grid, tickets and exchange as
the real kernel but no row traffic.  It must finish without an exchange
timeout, take longer with more row waves per cluster, and cost less than
the real kernel on the same shape."""
import pytest

from wide_reduction_reuse_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [(op, p) for op in W.OPS for p in (2, 4, 8)]


@pytest.mark.parametrize("op,p", CASES)
def test_control_kernel(op, p):
    import torch
    from wide_reduction_reuse_amd import credit as C
    from wide_reduction_reuse_amd import sweep
    from wide_reduction_reuse_amd.ctrlbench import time_control
    from wide_reduction_reuse_amd.timing import HipEvents
    assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
    cols = 65536
    plan = C.credit_plan(op, "f32", 64, cols, "split", p)
    occ = C.credit_occupancy(op, "f32", cols, plan)
    clusters = max(1, occ * torch.cuda.get_device_properties(0).multi_processor_count // p)
    t1 = time_control(C, HipEvents, op, clusters, cols, plan, 10, 2)
    t8 = time_control(C, HipEvents, op, clusters * 8, cols, plan, 10, 2)
    print("control %s P=%d %dx%d: 1 wave %.2f us, 8 waves %.2f us" % (op, p, plan.block_threads, plan.items, t1, t8),
          flush=True)
    assert t8 > t1
    # the real kernel on the same 8-wave shape moves every row; the control moves none
    w = W.custom(op, "f32", clusters * 8, cols, seed=3)
    t = sweep.device_inputs(w)
    ev = HipEvents(3)
    try:
        for i in range(3):
            C.credit_run_plan_timed(op, plan, t, *ev.pairs[i], eps=w.eps)
        torch.cuda.synchronize()
        C.credit_check_errors()
        real = ev.elapsed_ms(2) * 1000.0
    finally:
        ev.close()
    print("  real kernel %.2f us" % real, flush=True)
    assert t8 < real
