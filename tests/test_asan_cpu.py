"""The library's host code under AddressSanitizer, on the CPU.

A child process loads the host-ASan build of the library (libcredit_asan.so,
built by `python -m wide_reduction_reuse_amd.build --asan` and by
__graft_entry__.build(); the interpreter is not instrumented, so the
sanitizer runtime is preloaded) and drives every host path that runs without
a GPU: argument validation of every entry point, the selector and plan
enumeration over a grid of shapes with and without the shipped calibration,
forced and illegal plans, and the calibration parser on well-formed,
truncated and malformed files.  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import ctypes, json, os, sys, tempfile
sys.path.insert(0, sys.argv[1])
from wide_reduction_reuse_amd import credit as C
L = C.lib()
assert C.LIB_PATH.endswith("libcredit_asan.so"), C.LIB_PATH
ops = list(C.OPS)
shapes = [(0, 1), (1, 1), (3, 7), (64, 4096), (4096, 8192), (1024, 65536), (256, 262144), (33, 50257),
          (6, 100003), (2670, 50257), (1 << 20, 1024), (5, 1 << 22), (9000, 131072), (7, 20002)]
def grid():
    n = 0
    for op in ops:
        for dt in ("f32", "bf16"):
            for rows, cols in shapes:
                for path in ("auto", "single", "split", "reread"):
                    for p in (0, 2, 4, 8):
                        try:
                            pl = C.credit_plan(op, dt, rows, cols, path, p)
                            n += 1
                            C.credit_occupancy  # host-only below
                        except C.CreditError as e:
                            assert e.status in (1, 2, 4), (op, dt, rows, cols, path, p, e.status)
                for p in (2, 4, 8):
                    try:
                        C.credit_model_terms(op, dt, max(rows, 1), cols, p)
                    except C.CreditError as e:
                        assert e.status in (1, 2, 4), (op, dt, rows, cols, p, e.status)
                try:
                    C.credit_select_path(op, dt, rows, cols)
                    plans = C.credit_enumerate_plans(op, dt, rows, cols)
                    n += len(plans)
                except C.CreditError as e:
                    assert e.status in (1, 2, 4), (op, dt, rows, cols, e.status)
    return n
n1 = grid()                         # the shipped calibration
C.credit_load_calibration(None)     # the analytic model alone
n2 = grid()
# calibration parser: valid, truncated, malformed
good = open(C.CALIB_PATH).read()
bad = [good[: len(good) // 2], good[:10], "", "{", "[]", "{\"version\": 2, \"table\": [[0, 0]]}",
       "{\"version\": 2, \"table\": [[0,0,4096,1,1,64,2,16,-1,99,1,2]]}",
       "{\"version\": 2, \"table\": [[9,9,4096,1,1,64,2,16,-1,1,1,2]]}",
       "[" * 64 + "]" * 64, "{\"a\": \"\\", "{\"version\": 1e999}", "nul", "{\"version\": 2} trailing"]
for text in [good] + bad:
    with tempfile.NamedTemporaryFile("w", suffix=".json", delete=False) as f:
        f.write(text)
    st = L.credit_load_calibration(f.name.encode())
    os.unlink(f.name)
    assert st in (0, 6), st
assert L.credit_load_calibration(b"/nonexistent/calib.json") == 6
# argument validation of the operator entry points: errors before any HIP call
vp = ctypes.c_void_p
assert L.credit_softmax(None, None, 4, 16, 0, 0, 0, None) == 1
assert L.credit_softmax(vp(16), vp(32), -1, 16, 0, 0, 0, None) == 1
assert L.credit_softmax(vp(16), vp(32), 4, 0, 0, 0, 0, None) == 1
assert L.credit_softmax(vp(17), vp(32), 4, 16, 0, 0, 0, None) == 3
assert L.credit_softmax(vp(16), vp(32), 4, 16, 7, 0, 0, None) == 1
assert L.credit_softmax(vp(16), vp(32), 4, 16, 0, 9, 0, None) == 1
assert L.credit_softmax(vp(16), vp(32), 4, 16, 0, 2, 3, None) == 1
assert L.credit_layernorm(vp(16), None, vp(16), vp(32), 4, 16, ctypes.c_float(1e-5), 0, 0, 0, None) == 1
assert L.credit_layernorm(vp(16), vp(16), vp(16), vp(32), 4, 16, ctypes.c_float(-1.0), 0, 0, 0, None) == 1
assert L.credit_rmsnorm(vp(16), vp(16), vp(32), 4, 16, ctypes.c_float(float("nan")), 0, 0, 0, None) == 1
assert L.credit_layernorm_backward(vp(16), vp(16), vp(16), vp(32), 4, 16, ctypes.c_float(1e-5), 2, 0, 0, None) == 1
assert L.credit_quantize_int8(vp(16), vp(32), vp(2), 4, 16, 0, 0, 0, None) == 3
assert L.credit_softmax(vp(16), vp(32), 0, 16, 0, 0, 0, None) == 0  # rows = 0: a no-op
ops_t = C.Operands()
plan = C.Plan.make(2, 4, 1024, 16, 16)
assert L.credit_run_plan(0, ctypes.byref(ops_t), 4, 16, ctypes.c_float(0.0), 0, ctypes.byref(plan), None) == 1
assert L.credit_run_plan_static(0, ctypes.byref(ops_t), 4, 16, ctypes.c_float(0.0), 0, ctypes.byref(plan), None) == 1
assert L.credit_run_plan(0, None, 4, 16, ctypes.c_float(0.0), 0, None, None) == 1
assert L.credit_run_plan_timed(0, ctypes.byref(ops_t), 4, 16, ctypes.c_float(0.0), 0, ctypes.byref(plan), None, None, None) == 1
assert L.credit_control(0, 4, 16, 0, None, None, None, None) == 1
assert L.credit_copy(None, None, 16, None, None, None) == 1
assert L.credit_copy(vp(16), vp(32), 15, None, None, None) == 1
assert L.credit_flush(vp(8), 16, None) == 3
assert L.credit_select_path(0, 0, 4, 16, None) == 1
assert L.credit_enumerate_plans(0, 0, 4, 16, None, 3, None) == 1
n = ctypes.c_size_t()
assert L.credit_layernorm_backward_params_workspace(2048, 65536, 0, ctypes.byref(n)) == 0 and n.value > 0
assert L.credit_layernorm_backward_params_workspace(-1, 16, 0, ctypes.byref(n)) == 1
assert L.credit_layernorm_backward_params(None, None, None, None, None, 4, 16, 0, None, 0, None) == 1
assert L.credit_layernorm_backward_params(vp(16), vp(16), vp(16), vp(16), vp(16), 4, 16, 0, None, 0, None) == 1
assert L.credit_layernorm_backward_params(vp(17), vp(16), vp(16), vp(16), vp(16), 4, 16, 0, vp(16), 1 << 20, None) == 3
assert L.credit_layernorm_backward_stats(vp(16), vp(16), vp(16), vp(32), None, 4, 16, ctypes.c_float(1e-5), 0, 0, 0, None) == 1
assert L.credit_test_exchange(1 << 33) == 1
assert L.credit_test_exchange(-1) == 0
for s in range(-2, 12):
    assert L.credit_status_str(s)
assert L.credit_version() > 0
print("asan host paths ok: %d plans with the calibration, %d without" % (n1, n2))
'''


def test_host_code_under_address_sanitizer():
    from wide_reduction_reuse_amd import build as B
    if not os.path.exists(B.ASAN_LIB):
        pytest.skip("host-ASan library not built (python -m wide_reduction_reuse_amd.build --asan)")
    runtime = B.asan_runtime()
    if not runtime:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    env = dict(os.environ)
    env.update({"LD_PRELOAD": runtime, "CREDIT_LIB": B.ASAN_LIB, "CREDIT_CALIB": "",
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86:halt_on_error=1"})
    r = subprocess.run([sys.executable, "-c", SCRIPT, ROOT], env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=600)
    print(r.stdout[-2000:])
    assert "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    assert r.returncode == 0, r.stderr[-4000:]
    assert "asan host paths ok" in r.stdout
