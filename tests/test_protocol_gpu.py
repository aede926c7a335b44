"""The split-row exchange protocol on the GPU, through the C ABI: what happens
when a wait gives up, the restart of the exchange tags, graph capture and
replay, and split launches on two streams at once.

The protocol's state (ticket counter, tags) lives in each stream's scratch
and is advanced by the kernels themselves (the CREDIT paper protects the reuse
of its exchange buffers with a second cluster barrier per stage, Sec. III-C,
Eq. 5-6; here tags that never repeat between clears do it).  Failures are
forced from the host with the library's test hooks, so every kernel still
runs to its end: a reader that waits for a tag no workgroup writes gives up
after its poll limit, flags the error word and leaves NaN in the output.
"""
import numpy as np
import pytest

from wide_reduction_reuse_amd import workloads as W

from parity import check_result, from_device, to_device

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


def _operands(inp):
    import torch
    w = inp.workload
    t = W.alloc_outputs(w, {k: to_device(getattr(inp, k), w.dtype) for k in ("x", "dy", "gamma", "beta")})
    torch.cuda.synchronize()  # the uploads ran on the current stream; the tests use others
    return t


def _host(w, t):
    return {"y": from_device(t["y"], w.dtype),
            "row_out": None if t.get("row_out") is None else t["row_out"].cpu().numpy()}


def _check(inp, out, label):
    v = check_result(inp, out)
    print("%s: %s" % (label, v), flush=True)
    assert v.ok, "%s: %s" % (label, v)


def _all_nan(w, out):
    if w.op == "quantize_int8":
        return bool(np.isnan(out["row_out"]).all())
    y = out["y"]
    if w.dtype == "bf16":
        y = (y.astype(np.uint32) << 16).view(np.float32)
    return bool(np.isnan(y).all())


GIVE_UP_CASES = [("softmax", "f32"), ("softmax", "bf16"), ("layernorm", "bf16"), ("layernorm", "f32"),
                 ("rmsnorm", "f32"), ("rmsnorm", "bf16"), ("softmax_bwd", "f32"), ("layernorm_bwd", "f32"),
                 ("quantize_int8", "f32"), ("quantize_int8", "bf16")]


@pytest.mark.parametrize("p", [2, 4])
@pytest.mark.parametrize("op,dt", GIVE_UP_CASES)
def test_exchange_wait_that_gives_up_writes_nan_and_is_reported(op, dt, p):
    # Every reader waits for a tag no workgroup writes and gives up after its
    # first poll: the launch still ends, every row comes out NaN (the
    # quantizer's scales NaN), and credit_check_errors reports the timeout
    # once.  The same scratch then serves a normal launch correctly.
    import torch
    C = _lib()
    s = torch.cuda.Stream()
    w = W.custom(op, dt, 70, 8192, seed=101 + p, x_dist="scaled_shifted", x_scale=2.0, x_shift=0.5)
    inp = W.generate(w)
    t = _operands(inp)
    try:
        C.credit_test_exchange(0)
        C.credit_test_scratch(-1, True, stream=s)
        C.run(op, t, inp.eps, path="split", split_p=p, stream=s)
        with pytest.raises(C.CreditError) as ei:
            C.credit_check_errors(s)
        assert ei.value.status == 8  # CREDIT_ERR_DEVICE_TIMEOUT
    finally:
        C.credit_test_exchange(-1)
        C.credit_test_scratch(-1, False, stream=s)
    C.credit_check_errors(s)  # reported once, then clear
    out = _host(w, t)
    assert _all_nan(w, out), "a row written from stale statistics"
    C.run(op, t, inp.eps, path="split", split_p=p, stream=s, check=True)
    _check(inp, _host(w, t), "after give-up %s %s P=%d" % (op, dt, p))


@pytest.mark.parametrize("op,dt,p", [("softmax", "f32", 8), ("layernorm", "bf16", 4), ("softmax_bwd", "f32", 2)])
def test_tag_restart_clears_stale_words(op, dt, p):
    # Three times: (a) 100 rows, one row per cluster, leave words with tag 1
    # in 100 clusters' slots, from inputs offset by +1000; (b) with the tag
    # count set just below the restart point, a launch of 10 rows crosses it:
    # its last workgroup clears every word and restarts the tags; (c) the
    # 100-row shape again, on inputs without the offset, expects tag 1 from
    # each peer.  Had the words of (a) survived in the 90 clusters (b) did not
    # touch, a reader that polls before its peer has written would take (a)'s
    # statistics, 1000 off.  Then (c) again, at tag 2, and the many-row case.
    import torch
    C = _lib()
    s = torch.cuda.Stream()
    cols = 256 if dt == "f32" else 512
    for cycle in range(3):
        seed = 200 + 10 * cycle
        a = W.generate(W.custom(op, dt, 100, cols, seed=seed, x_dist="scaled_shifted", x_scale=3.0,
                                x_shift=1000.0))
        b = W.generate(W.custom(op, dt, 10, cols, seed=seed + 1))
        c = W.generate(W.custom(op, dt, 100, cols, seed=seed + 2, x_dist="scaled_shifted", x_scale=3.0,
                                x_shift=0.5))
        ta, tb, tc = _operands(a), _operands(b), _operands(c)
        C.run(op, ta, a.eps, path="split", split_p=p, stream=s, check=True)
        _check(a, _host(a.workload, ta), "tags (a) %s cycle %d" % (op, cycle))
        C.credit_test_scratch((1 << 31) - 1, False, stream=s)
        C.run(op, tb, b.eps, path="split", split_p=p, stream=s, check=True)
        _check(b, _host(b.workload, tb), "tags (b), crossing the restart, %s cycle %d" % (op, cycle))
        for rep in range(2):
            C.run(op, tc, c.eps, path="split", split_p=p, stream=s, check=True)
            _check(c, _host(c.workload, tc), "tags (c%d) after the restart %s cycle %d" % (rep, op, cycle))
    many = W.generate(W.custom(op, dt, 40000, cols, seed=299, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5))
    tm = _operands(many)
    C.credit_test_scratch((1 << 31) - 5, False, stream=s)
    for rep in range(2):  # issues tags past 2^31 and restarts them at its end; then from tag 1
        C.run(op, tm, many.eps, path="split", split_p=p, stream=s, check=True)
        _check(many, _host(many.workload, tm), "tags, many rows, rep %d %s" % (rep, op))
    torch.cuda.synchronize()


GRAPH_CASES = [("softmax", "f32", 64, 262144, 4), ("layernorm", "bf16", 300, 65536, 2),
               ("quantize_int8", "f32", 100, 65536, 2), ("softmax_bwd", "f32", 40, 65536, 2)]


@pytest.mark.parametrize("op,dt,rows,cols,p", GRAPH_CASES)
def test_split_launch_captured_in_a_graph_replays_correctly(op, dt, rows, cols, p):
    # Capture one split launch, then replay it three times on new inputs
    # (copied into the captured buffers), with eager split launches on the
    # same stream and synchronizations between the replays; every replay
    # must match the oracle on its own inputs.
    import torch
    C = _lib()
    s = torch.cuda.Stream()
    w = W.custom(op, dt, rows, cols, seed=300, x_dist="scaled_shifted", x_scale=3.0, x_shift=0.5)
    inp0 = W.generate(w)
    t = _operands(inp0)
    other = W.generate(W.custom(op, dt, 33, cols, seed=399))
    t_other = _operands(other)
    C.run(op, t, inp0.eps, path="split", split_p=p, stream=s, check=True)  # creates the stream's scratch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        C.run(op, t, inp0.eps, path="split", split_p=p)
    torch.cuda.synchronize()
    for i in range(3):
        inp = W.generate(W.custom(op, dt, rows, cols, seed=301 + i, x_dist="scaled_shifted", x_scale=3.0,
                                  x_shift=0.5))
        for k in ("x", "dy", "gamma", "beta"):
            if t.get(k) is not None:
                t[k].copy_(to_device(getattr(inp, k), w.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        C.credit_check_errors(s)
        _check(inp, _host(w, t), "graph replay %d %s %s P=%d" % (i, op, dt, p))
        C.run(op, t_other, other.eps, path="split", split_p=p, stream=s, check=True)
        _check(other, _host(other.workload, t_other), "eager between replays %s" % op)
    del g
    torch.cuda.synchronize()


def test_first_split_call_under_capture_is_refused():
    # The scratch of a stream is allocated on its first split-row call, which
    # cannot be captured: the call returns CREDIT_ERR_UNSUPPORTED and
    # enqueues nothing.
    import torch
    C = _lib()
    s = torch.cuda.Stream()
    x = torch.randn(8, 65536, device="cuda")
    y = torch.empty_like(x)
    # the same plan on the current stream first, so that the library has
    # queried everything else it needs (occupancy) outside the capture
    C.credit_softmax(x, y, "split", 4, check=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(C.CreditError) as ei:
            C.credit_softmax(x, y, "split", 4)
    assert ei.value.status == 2
    del g
    torch.cuda.synchronize()


def test_split_launches_on_two_streams_at_once():
    # Two streams, each with its own scratch, each enqueuing split launches
    # back to back without synchronizing in between, so that they run
    # concurrently; every result matches the oracle.
    import torch
    C = _lib()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cases = [W.custom("softmax", "f32", 64, 262144, seed=401, x_dist="row_offset", x_scale=4.0, row_offset=50.0),
             W.custom("layernorm", "bf16", 600, 65536, seed=402, x_dist="scaled_shifted", x_scale=3.0,
                      x_shift=0.5)]
    splits = [4, 2]
    inps = [W.generate(w) for w in cases]
    ts = [[_operands(inp) for _ in range(3)] for inp in inps]
    for rep in range(3):
        for j in range(2):
            C.run(cases[j].op, ts[j][rep], inps[j].eps, path="split", split_p=splits[j], stream=streams[j])
    for j in range(2):
        C.credit_check_errors(streams[j])
    for j in range(2):
        for rep in range(3):
            _check(inps[j], _host(cases[j], ts[j][rep]), "two streams: %s rep %d" % (cases[j].name, rep))
