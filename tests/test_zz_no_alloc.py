"""credit_run_plan_static, the entry point that allocates no device memory,
against credit_run_plan on the same plans and inputs, through the C ABI.

Both run the same kernels; only the split-row exchange scratch differs (the
library's static array instead of the stream's allocated scratch).  For each
case two calls follow each other, the second on fewer rows: the outputs of
the two entry points must be identical, and within the oracle's tolerance.
Then a first call on a fresh stream is captured into a graph and replayed on
new inputs.
"""
import numpy as np
import pytest

from wide_reduction_reuse_amd import workloads as W

from parity import check_result, from_device, to_device

pytestmark = pytest.mark.gpu

# (op, dtype, cols, path, P, rows of the first call, rows of the second)
CASES = [("softmax", "f32", 65536, "split", 2, 600, 7),
         ("softmax", "f32", 262144, "split", 4, 256, 3),
         ("layernorm", "bf16", 65536, "split", 2, 900, 5),
         ("rmsnorm", "bf16", 131072, "split", 8, 500, 9),
         ("softmax_bwd", "f32", 65536, "split", 2, 300, 4),
         ("layernorm_bwd", "f32", 65536, "split", 2, 300, 3),
         ("quantize_int8", "f32", 65536, "split", 4, 400, 2),
         ("softmax", "bf16", 50257, "split", 4, 300, 5),
         ("layernorm", "bf16", 8192, "single", 0, 4096, 11),
         ("rmsnorm", "f32", 16384, "reread", 0, 300, 5)]


def _lib():
    import torch
    from wide_reduction_reuse_amd import credit
    assert torch.cuda.is_available(), "GPU test selected but no GPU is visible"
    return credit


def _operands(inp):
    w = inp.workload
    return W.alloc_outputs(w, {k: to_device(getattr(inp, k), w.dtype) for k in ("x", "dy", "gamma", "beta")})


def _host(w, t):
    return {"y": from_device(t["y"], w.dtype),
            "row_out": None if t.get("row_out") is None else t["row_out"].cpu().numpy()}


@pytest.mark.parametrize("op,dt,cols,path,p,rows1,rows2", CASES,
                         ids=["%s-%s-c%d-%s%d" % c[:5] for c in CASES])
def test_static_entry_matches_run_plan(op, dt, cols, path, p, rows1, rows2):
    import torch
    C = _lib()
    for i, rows in enumerate((rows1, rows2)):
        w = W.custom(op, dt, rows, cols, seed=500 + 17 * i + cols % 97, x_dist="scaled_shifted", x_scale=3.0,
                     x_shift=0.5)
        inp = W.generate(w)
        plan = C.credit_plan(op, dt, rows, cols, path, p)
        t_ref = _operands(inp)
        t_static = W.alloc_outputs(w, {k: t_ref[k] for k in ("x", "dy", "gamma", "beta")})
        C.credit_run_plan(op, plan, t_ref, eps=inp.eps, check=True)
        C.credit_run_plan_static(op, plan, t_static, eps=inp.eps, check=True)
        torch.cuda.synchronize()
        ref, got = _host(w, t_ref), _host(w, t_static)
        assert np.array_equal(ref["y"], got["y"]), "call %d: outputs differ from credit_run_plan" % i
        if ref["row_out"] is not None:
            assert np.array_equal(ref["row_out"].view(np.uint32), got["row_out"].view(np.uint32))
        v = check_result(inp, got)
        print("static %s %s %dx%d %s P=%d: %s" % (op, dt, rows, cols, path, p, v), flush=True)
        assert v.ok, str(v)


def test_static_entry_first_call_on_a_stream_captured_and_replayed():
    # The stream has never run a split-row call, so credit_run_plan would
    # have to allocate its scratch and refuses under capture; the static
    # entry point needs none.  Three replays on new inputs, each checked.
    import torch
    C = _lib()
    op, dt, rows, cols, p = "softmax", "f32", 64, 262144, 4
    w = W.custom(op, dt, rows, cols, seed=600, x_dist="row_offset", x_scale=4.0, row_offset=50.0)
    inp = W.generate(w)
    t = _operands(inp)
    plan = C.credit_plan(op, dt, rows, cols, "split", p)
    C.credit_run_plan_static(op, plan, t, eps=inp.eps, check=True)  # module and symbol set up uncaptured
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        C.credit_run_plan_static(op, plan, t, eps=inp.eps)
    torch.cuda.synchronize()
    for i in range(3):
        inp_i = W.generate(W.custom(op, dt, rows, cols, seed=601 + i, x_dist="row_offset", x_scale=4.0,
                                    row_offset=50.0))
        t["x"].copy_(to_device(inp_i.x, dt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C.credit_check_errors()
        v = check_result(inp_i, _host(w, t))
        print("static graph replay %d: %s" % (i, v), flush=True)
        assert v.ok, str(v)
    del g
    torch.cuda.synchronize()
