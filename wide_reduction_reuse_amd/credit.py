"""Thin ctypes binding to libcredit.so (include/credit.h).

Argument marshalling only: tensors are passed as device pointers, the stream as
torch's current HIP stream.  Every computation runs in the library's kernels;
if the library has not been built this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# CREDIT_LIB may name another build of the library (the host-ASan variant)
LIB_PATH = os.environ.get("CREDIT_LIB") or os.path.join(PKG, "libcredit.so")
# selector calibration measured on MI355X, loaded with the library unless
# CREDIT_CALIB names another file (the library then loads that one itself)
CALIB_PATH = os.path.join(PKG, "calib", "mi355x.json")

# status codes (credit_status_t)
OK = 0
STATUS_NAMES = {0: "CREDIT_OK", 1: "CREDIT_ERR_INVALID_ARG", 2: "CREDIT_ERR_UNSUPPORTED",
                3: "CREDIT_ERR_ALIGNMENT", 4: "CREDIT_ERR_ILLEGAL_PATH", 5: "CREDIT_ERR_NOT_CORESIDENT",
                6: "CREDIT_ERR_NO_CALIBRATION", 7: "CREDIT_ERR_HIP", 8: "CREDIT_ERR_DEVICE_TIMEOUT"}
# dtypes, ops, paths
F32, BF16 = 0, 1
SOFTMAX, LAYERNORM, RMSNORM, SOFTMAX_BACKWARD, LAYERNORM_BACKWARD, QUANTIZE_INT8 = 0, 1, 2, 3, 4, 5
PATH_AUTO, PATH_SINGLE_WG, PATH_SPLIT_ROW, PATH_REREAD = 0, 1, 2, 3
PATHS = {"auto": 0, "single": 1, "split": 2, "reread": 3}
OPS = {"softmax": 0, "layernorm": 1, "rmsnorm": 2, "softmax_bwd": 3, "layernorm_bwd": 4, "quantize_int8": 5}
DTYPES = {"f32": 0, "bf16": 1}
# operands each operator reads or writes (credit_operands_t)
OPERANDS = {"softmax": ("x", "y"), "layernorm": ("x", "gamma", "beta", "y"), "rmsnorm": ("x", "gamma", "y"),
            "softmax_bwd": ("x", "dy", "y"), "layernorm_bwd": ("x", "dy", "gamma", "y"),
            "quantize_int8": ("x", "y", "row_out")}

EXPORTED = ["credit_softmax", "credit_layernorm", "credit_rmsnorm", "credit_softmax_backward",
            "credit_layernorm_backward", "credit_quantize_int8", "credit_select_path", "credit_make_plan",
            "credit_enumerate_plans", "credit_occupancy",
            "credit_run_plan", "credit_run_plan_timed", "credit_run_plan_static", "credit_control", "credit_copy",
            "credit_flush", "credit_load_calibration", "credit_check_errors", "credit_status_str", "credit_version",
            "credit_test_exchange", "credit_test_scratch", "credit_model_terms",
            "credit_layernorm_backward_stats", "credit_layernorm_backward_params",
            "credit_layernorm_backward_params_workspace"]


class CreditError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, STATUS_NAMES.get(status, "?"), status))


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_p", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("items", ctypes.c_int32), ("vec_bytes", ctypes.c_int32), ("wgs_per_cu", ctypes.c_int32),
                ("lds_items", ctypes.c_int32), ("predicted_us", ctypes.c_double * 3)]

    def as_dict(self) -> dict:
        return {"path": self.path, "split_p": self.split_p, "block_threads": self.block_threads,
                "items": self.items, "vec_bytes": self.vec_bytes, "wgs_per_cu": self.wgs_per_cu,
                "lds_items": self.lds_items, "predicted_us": [self.predicted_us[i] for i in range(3)]}

    @classmethod
    def make(cls, path: int, split_p: int, block_threads: int, items: int, vec_bytes: int = 0,
             wgs_per_cu: int = 0, lds_items: int = 0) -> "Plan":
        p = cls()
        p.path, p.split_p, p.block_threads, p.items, p.vec_bytes = path, split_p, block_threads, items, vec_bytes
        p.wgs_per_cu, p.lds_items = wgs_per_cu, lds_items
        return p


class ModelTerms(ctypes.Structure):
    _fields_ = [("baseline_path", ctypes.c_int32), ("split_block", ctypes.c_int32),
                ("split_items", ctypes.c_int32), ("split_resident", ctypes.c_int32)] + \
               [(k, ctypes.c_double) for k in ("t_base_us", "b_base", "b_reread", "t_save_us", "t_occ_us", "waves",
                                               "t_ctrl_us", "t_dsm_us", "delta_us", "t_split_us")]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class Operands(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dy", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("y", ctypes.c_void_p), ("row_out", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcredit.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libcredit.so is not built (run `python -m wide_reduction_reuse_amd.build`); "
                           "there is no fallback implementation")
    # torch bundles its own HIP runtime under the same soname; loading torch
    # first makes libcredit.so bind to that one copy rather than a second one
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    sig = {
        "credit_softmax": [vp, vp, i64, i64, i32, i32, i32, vp],
        "credit_layernorm": [vp, vp, vp, vp, i64, i64, f32, i32, i32, i32, vp],
        "credit_rmsnorm": [vp, vp, vp, i64, i64, f32, i32, i32, i32, vp],
        "credit_softmax_backward": [vp, vp, vp, i64, i64, i32, i32, i32, vp],
        "credit_layernorm_backward": [vp, vp, vp, vp, i64, i64, f32, i32, i32, i32, vp],
        "credit_layernorm_backward_stats": [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, i32, vp],
        "credit_layernorm_backward_params": [vp, vp, vp, vp, vp, i64, i64, i32, vp, ctypes.c_size_t, vp],
        "credit_layernorm_backward_params_workspace": [i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)],
        "credit_quantize_int8": [vp, vp, vp, i64, i64, i32, i32, i32, vp],
        "credit_select_path": [i32, i32, i64, i64, ctypes.POINTER(Plan)],
        "credit_make_plan": [i32, i32, i64, i64, i32, i32, ctypes.POINTER(Plan)],
        "credit_enumerate_plans": [i32, i32, i64, i64, ctypes.POINTER(Plan), i32, ctypes.POINTER(i32)],
        "credit_occupancy": [i32, i32, i64, ctypes.POINTER(Plan), ctypes.POINTER(i32)],
        "credit_run_plan": [i32, ctypes.POINTER(Operands), i64, i64, f32, i32, ctypes.POINTER(Plan), vp],
        "credit_run_plan_timed": [i32, ctypes.POINTER(Operands), i64, i64, f32, i32, ctypes.POINTER(Plan), vp, vp,
                                  vp],
        "credit_run_plan_static": [i32, ctypes.POINTER(Operands), i64, i64, f32, i32, ctypes.POINTER(Plan), vp],
        "credit_control": [i32, i64, i64, i32, ctypes.POINTER(Plan), vp, vp, vp],
        "credit_copy": [vp, vp, i64, vp, vp, vp],
        "credit_flush": [vp, i64, vp],
        "credit_load_calibration": [ctypes.c_char_p],
        "credit_check_errors": [vp],
        "credit_status_str": [i32],
        "credit_version": [],
        "credit_test_exchange": [i64],
        "credit_test_scratch": [i64, i32, vp],
        "credit_model_terms": [i32, i32, i64, i64, i32, ctypes.POINTER(ModelTerms)],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int32
    L.credit_status_str.restype = ctypes.c_char_p
    if not os.environ.get("CREDIT_CALIB") and os.path.exists(CALIB_PATH):
        status = L.credit_load_calibration(CALIB_PATH.encode())
        if status != OK:
            raise CreditError(status, "credit_load_calibration(%s)" % CALIB_PATH)
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != OK:
        raise CreditError(status, where)


def _finish(check: bool, stream) -> None:
    """With check=True: synchronize the stream and raise if a split-row
    exchange wait gave up (credit_check_errors), whose rows were written as NaN."""
    if check:
        credit_check_errors(stream)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _shape2d(x):
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    cols = x.shape[-1] if x.dim() else 1
    rows = x.numel() // cols if cols else 0
    return rows, cols


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _path(path) -> int:
    return PATHS[path] if isinstance(path, str) else int(path)


def _out(x, y, dtype=None):
    import torch
    dtype = x.dtype if dtype is None else dtype
    if y is None:
        y = torch.empty(x.shape, dtype=dtype, device=x.device)
    if y.shape != x.shape or y.dtype != dtype or not y.is_contiguous():
        raise ValueError("the output must be a contiguous %s tensor with x's shape" % dtype)
    return y


def _same(x, t, name):
    if t.shape != x.shape or t.dtype != x.dtype or not t.is_contiguous():
        raise ValueError("%s must be a contiguous tensor with x's shape and dtype" % name)


def credit_softmax(x, y=None, path="auto", split_p: int = 0, stream=None, check: bool = False):
    y = _out(x, y)
    rows, cols = _shape2d(x)
    _check(lib().credit_softmax(_ptr(x), _ptr(y), rows, cols, _dtype_code(x), _path(path), split_p,
                                _stream(stream)), "credit_softmax")
    _finish(check, stream)
    return y


def credit_layernorm(x, gamma, beta, eps: float, y=None, path="auto", split_p: int = 0, stream=None,
                     check: bool = False):
    y = _out(x, y)
    rows, cols = _shape2d(x)
    _check(lib().credit_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), rows, cols, float(eps),
                                  _dtype_code(x), _path(path), split_p, _stream(stream)), "credit_layernorm")
    _finish(check, stream)
    return y


def credit_rmsnorm(x, gamma, eps: float, y=None, path="auto", split_p: int = 0, stream=None,
                   check: bool = False):
    y = _out(x, y)
    rows, cols = _shape2d(x)
    _check(lib().credit_rmsnorm(_ptr(x), _ptr(gamma), _ptr(y), rows, cols, float(eps), _dtype_code(x),
                                _path(path), split_p, _stream(stream)), "credit_rmsnorm")
    _finish(check, stream)
    return y


def credit_softmax_backward(x, dy, dx=None, path="auto", split_p: int = 0, stream=None, check: bool = False):
    """Gradient of row-wise softmax with respect to its logits x, given dy."""
    _same(x, dy, "dy")
    dx = _out(x, dx)
    rows, cols = _shape2d(x)
    _check(lib().credit_softmax_backward(_ptr(x), _ptr(dy), _ptr(dx), rows, cols, _dtype_code(x), _path(path),
                                         split_p, _stream(stream)), "credit_softmax_backward")
    _finish(check, stream)
    return dx


def credit_layernorm_backward(x, dy, gamma, eps: float, dx=None, path="auto", split_p: int = 0, stream=None,
                              check: bool = False):
    """Row part of the LayerNorm gradient: dL/dx given dL/dy (fp32)."""
    _same(x, dy, "dy")
    dx = _out(x, dx)
    rows, cols = _shape2d(x)
    _check(lib().credit_layernorm_backward(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(dx), rows, cols, float(eps),
                                           _dtype_code(x), _path(path), split_p, _stream(stream)),
           "credit_layernorm_backward")
    _finish(check, stream)
    return dx


def credit_layernorm_backward_stats(x, dy, gamma, eps: float, dx=None, stats=None, path="auto", split_p: int = 0,
                                    stream=None, check: bool = False):
    """credit_layernorm_backward, also writing each row's (mean, rstd): returns (dx, stats [rows][2] fp32)."""
    import torch
    _same(x, dy, "dy")
    dx = _out(x, dx)
    rows, cols = _shape2d(x)
    if stats is None:
        stats = torch.empty((rows, 2), dtype=torch.float32, device=x.device)
    if stats.numel() != 2 * rows or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError("stats must be a contiguous float32 tensor of two entries per row")
    _check(lib().credit_layernorm_backward_stats(_ptr(x), _ptr(dy), _ptr(gamma), _ptr(dx), _ptr(stats), rows, cols,
                                                 float(eps), _dtype_code(x), _path(path), split_p, _stream(stream)),
           "credit_layernorm_backward_stats")
    _finish(check, stream)
    return dx, stats


def credit_layernorm_backward_params_workspace(rows: int, cols: int, dtype) -> int:
    n = ctypes.c_size_t()
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib().credit_layernorm_backward_params_workspace(rows, cols, dt, ctypes.byref(n)),
           "credit_layernorm_backward_params_workspace")
    return n.value


def credit_layernorm_backward_params(x, dy, stats, dgamma=None, dbeta=None, workspace=None, stream=None):
    """Parameter part of the LayerNorm gradient: returns (dgamma, dbeta), fp32 [cols].
    `stats` as credit_layernorm_backward_stats returns them; the workspace is
    allocated when not given."""
    import torch
    _same(x, dy, "dy")
    rows, cols = _shape2d(x)
    if dgamma is None:
        dgamma = torch.empty(cols, dtype=torch.float32, device=x.device)
    if dbeta is None:
        dbeta = torch.empty(cols, dtype=torch.float32, device=x.device)
    for name, v in (("dgamma", dgamma), ("dbeta", dbeta)):
        if v.numel() != cols or v.dtype != torch.float32 or not v.is_contiguous():
            raise ValueError("%s must be a contiguous float32 tensor of cols entries" % name)
    need = credit_layernorm_backward_params_workspace(rows, cols, _dtype_code(x))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().credit_layernorm_backward_params(_ptr(x), _ptr(dy), _ptr(stats), _ptr(dgamma), _ptr(dbeta), rows,
                                                  cols, _dtype_code(x), _ptr(workspace), workspace.numel(),
                                                  _stream(stream)), "credit_layernorm_backward_params")
    return dgamma, dbeta


def credit_quantize_int8(x, q=None, scale=None, path="auto", split_p: int = 0, stream=None, check: bool = False):
    """Row-wise symmetric int8 quantization: returns (q int8 like x, scale float32 [rows])."""
    import torch
    q = _out(x, q, torch.int8)
    rows, cols = _shape2d(x)
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if scale.numel() != rows or scale.dtype != torch.float32 or not scale.is_contiguous():
        raise ValueError("scale must be a contiguous float32 tensor with one entry per row")
    _check(lib().credit_quantize_int8(_ptr(x), _ptr(q), _ptr(scale), rows, cols, _dtype_code(x), _path(path),
                                      split_p, _stream(stream)), "credit_quantize_int8")
    _finish(check, stream)
    return q, scale


def credit_select_path(op, dtype, rows: int, cols: int) -> Plan:
    p = Plan()
    op = OPS[op] if isinstance(op, str) else int(op)
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib().credit_select_path(op, dt, rows, cols, ctypes.byref(p)), "credit_select_path")
    return p


def credit_plan(op, dtype, rows: int, cols: int, path="auto", split_p: int = 0) -> Plan:
    """credit_make_plan: the plan the entry points use for a (possibly forced) path."""
    p = Plan()
    op = OPS[op] if isinstance(op, str) else int(op)
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib().credit_make_plan(op, dt, rows, cols, _path(path), split_p, ctypes.byref(p)), "credit_make_plan")
    return p


def credit_model_terms(op, dtype, rows: int, cols: int, split_p: int) -> ModelTerms:
    """The analytic model's Eq. 7-9 terms for splitting the shape P ways."""
    t = ModelTerms()
    op = OPS[op] if isinstance(op, str) else int(op)
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib().credit_model_terms(op, dt, rows, cols, split_p, ctypes.byref(t)), "credit_model_terms")
    return t


def credit_enumerate_plans(op, dtype, rows: int, cols: int):
    """Every legal plan for the shape (credit_enumerate_plans), as a list of Plan."""
    op = OPS[op] if isinstance(op, str) else int(op)
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    n = ctypes.c_int32()
    _check(lib().credit_enumerate_plans(op, dt, rows, cols, None, 0, ctypes.byref(n)), "credit_enumerate_plans")
    arr = (Plan * max(1, n.value))()
    _check(lib().credit_enumerate_plans(op, dt, rows, cols, arr, n.value, ctypes.byref(n)),
           "credit_enumerate_plans")
    return [arr[i] for i in range(n.value)]


def credit_occupancy(op, dtype, cols: int, plan: Plan) -> int:
    """Resident workgroups per CU of the kernel `plan` selects (credit_occupancy)."""
    op = OPS[op] if isinstance(op, str) else int(op)
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    n = ctypes.c_int32()
    _check(lib().credit_occupancy(op, dt, cols, ctypes.byref(plan), ctypes.byref(n)), "credit_occupancy")
    return n.value


def operands(t) -> Operands:
    """credit_operands_t from a mapping with keys among x, dy, gamma, beta, y,
    row_out (tensors or None)."""
    o = Operands()
    for k in ("x", "dy", "gamma", "beta", "y", "row_out"):
        v = t.get(k)
        setattr(o, k, None if v is None else v.data_ptr())
    return o


def credit_run_plan(op, plan: Plan, t, eps: float = 0.0, stream=None, check: bool = False):
    """Run `plan` on the operands in mapping `t` (see operands())."""
    op = OPS[op] if isinstance(op, str) else int(op)
    rows, cols = _shape2d(t["x"])
    o = operands(t)
    _check(lib().credit_run_plan(op, ctypes.byref(o), rows, cols, float(eps), _dtype_code(t["x"]),
                                 ctypes.byref(plan), _stream(stream)), "credit_run_plan")
    _finish(check, stream)
    return t["y"]


def credit_run_plan_static(op, plan: Plan, t, eps: float = 0.0, stream=None, check: bool = False):
    """credit_run_plan on the library's static split-row scratch: allocates no
    device memory (for graph capture and serving loops)."""
    op = OPS[op] if isinstance(op, str) else int(op)
    rows, cols = _shape2d(t["x"])
    o = operands(t)
    _check(lib().credit_run_plan_static(op, ctypes.byref(o), rows, cols, float(eps), _dtype_code(t["x"]),
                                        ctypes.byref(plan), _stream(stream)), "credit_run_plan_static")
    _finish(check, stream)
    return t["y"]


def credit_run_plan_timed(op, plan: Plan, t, start_event: int, stop_event: int, eps: float = 0.0, stream=None):
    """credit_run_plan with timing; start_event / stop_event: raw hipEvent_t handles (integers)."""
    op = OPS[op] if isinstance(op, str) else int(op)
    rows, cols = _shape2d(t["x"])
    o = operands(t)
    _check(lib().credit_run_plan_timed(op, ctypes.byref(o), rows, cols, float(eps), _dtype_code(t["x"]),
                                       ctypes.byref(plan), ctypes.c_void_p(start_event),
                                       ctypes.c_void_p(stop_event), _stream(stream)), "credit_run_plan_timed")
    return t["y"]


def credit_control(op, rows: int, cols: int, dtype, plan: Plan, start_event: Optional[int] = None,
                   stop_event: Optional[int] = None, stream=None) -> None:
    """The work-free control kernel of a split plan; the events (raw hipEvent_t
    handles, optional) take its dispatch timestamps."""
    op = OPS[op] if isinstance(op, str) else int(op)
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib().credit_control(op, rows, cols, dt, ctypes.byref(plan), ctypes.c_void_p(start_event),
                                ctypes.c_void_p(stop_event), _stream(stream)), "credit_control")


def credit_copy(src, dst, start_event: Optional[int] = None, stop_event: Optional[int] = None,
                stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    _check(lib().credit_copy(_ptr(src), _ptr(dst), nbytes, ctypes.c_void_p(start_event),
                             ctypes.c_void_p(stop_event), _stream(stream)), "credit_copy")


def credit_flush(buf, stream=None) -> None:
    nbytes = buf.numel() * buf.element_size()
    _check(lib().credit_flush(_ptr(buf), nbytes, _stream(stream)), "credit_flush")


def credit_load_calibration(path: Optional[str]) -> None:
    _check(lib().credit_load_calibration(None if path is None else path.encode()), "credit_load_calibration")


def credit_check_errors(stream=None) -> None:
    _check(lib().credit_check_errors(_stream(stream)), "credit_check_errors")


def credit_test_exchange(spin_limit: int = -1) -> None:
    """Test hook: polls before a split-row exchange wait gives up (-1 = default)."""
    _check(lib().credit_test_exchange(int(spin_limit)), "credit_test_exchange")


def credit_test_scratch(tags_used: int, unmatched_tags: bool = False, stream=None) -> None:
    """Test hook: set the exchange-tag count of the stream's split-row scratch
    (tags_used < 0 leaves it) and, with unmatched_tags, make every exchange
    wait give up."""
    _check(lib().credit_test_scratch(int(tags_used), 1 if unmatched_tags else 0, _stream(stream)),
           "credit_test_scratch")


def credit_status_str(status: int) -> str:
    return lib().credit_status_str(status).decode()


def credit_version() -> int:
    return int(lib().credit_version())


def run(op: str, t, eps: float = 0.0, path="auto", split_p: int = 0, stream=None, check: bool = False):
    """Dispatch by operator name to the matching entry point.  `t` maps operand
    names (x, dy, gamma, beta; outputs y and row_out, allocated when absent)
    to tensors.  Returns the output row tensor (for quantization, (q, scale)).
    check=True synchronizes and raises CreditError if a split-row exchange
    wait gave up."""
    x = t["x"]
    y = t.get("y")
    if op == "softmax":
        return credit_softmax(x, y, path, split_p, stream, check)
    if op == "layernorm":
        return credit_layernorm(x, t["gamma"], t["beta"], eps, y, path, split_p, stream, check)
    if op == "rmsnorm":
        return credit_rmsnorm(x, t["gamma"], eps, y, path, split_p, stream, check)
    if op == "softmax_bwd":
        return credit_softmax_backward(x, t["dy"], y, path, split_p, stream, check)
    if op == "layernorm_bwd":
        return credit_layernorm_backward(x, t["dy"], t["gamma"], eps, y, path, split_p, stream, check)
    if op == "quantize_int8":
        return credit_quantize_int8(x, y, t.get("row_out"), path, split_p, stream, check)
    raise ValueError(op)
