"""ctypes binding of librmsnorm_mi355x.so (include/rmsnorm.h).

Argument marshalling only: every step of the forward runs in the HIP kernels.
PyTorch provides device memory and the current stream.  If the library is not
built, importing this module raises; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "librmsnorm_mi355x.so")

RMSNORM_BF16 = 0
RMSNORM_FP16 = 1
RMSNORM_FP32 = 2          # forward only
DTYPE_CODES = {torch.bfloat16: RMSNORM_BF16, torch.float16: RMSNORM_FP16, torch.float32: RMSNORM_FP32}
DTYPE_NAMES = {"bf16": RMSNORM_BF16, "fp16": RMSNORM_FP16, "fp32": RMSNORM_FP32}

VARIANT_AUTO, VARIANT_WAVE, VARIANT_BLOCK, VARIANT_GENERIC, VARIANT_SHIFTED, VARIANT_SHIFTED_WAVE, VARIANT_WIDE = \
    0, 1, 2, 3, 4, 5, 6
VARIANT_NAMES = {VARIANT_WAVE: "wave", VARIANT_BLOCK: "block", VARIANT_GENERIC: "generic",
                 VARIANT_SHIFTED: "shifted", VARIANT_SHIFTED_WAVE: "shifted_wave", VARIANT_WIDE: "wide"}

STATUS = {
    0: "RMSNORM_OK", 1: "RMSNORM_ERR_NULL", 2: "RMSNORM_ERR_SHAPE", 3: "RMSNORM_ERR_DTYPE",
    4: "RMSNORM_ERR_SCALAR", 5: "RMSNORM_ERR_OVERLAP", 6: "RMSNORM_ERR_HIP",
    7: "RMSNORM_ERR_DEVICE", 8: "RMSNORM_ERR_PLAN",
}

# Every symbol include/rmsnorm.h declares.
EXPORTED = (
    "rmsnorm_fwd", "rmsnorm_fwd_with_plan", "rmsnorm_fwd_ex", "rmsnorm_plan_query", "rmsnorm_plan_query_ex",
    "rmsnorm_plan_resources", "rmsnorm_fwd_kernel_query",
    "rmsnorm_bwd", "rmsnorm_bwd_with_plan", "rmsnorm_bwd_plan_query", "rmsnorm_bwd_workspace_size",
    "rmsnorm_bwd_plan_validate",
    "rmsnorm_bwd_noalloc",
    "rmsnorm_bwd_ex", "rmsnorm_bwd_plan_query_ex", "rmsnorm_bwd_workspace_size_ex",
    "rmsnorm_plan_validate", "rmsnorm_plan_set_tuned", "rmsnorm_plan_clear_tuned", "rmsnorm_plan_tuned_count",
    "rmsnorm_status_string", "rmsnorm_last_error", "rmsnorm_version",
)


class RmsnormError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = STATUS.get(status, f"status {status}")
        super().__init__(f"{name}: {detail}" if detail else name)


class Plan(ctypes.Structure):
    """rmsnorm_plan_t"""
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("vec_elems", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("vectors_per_lane", ctypes.c_int32),
        ("row_slots", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("prefetch", ctypes.c_int32),
        ("xcd_group", ctypes.c_int32),
        ("max_blocks_per_cu", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("rows_per_trip", ctypes.c_int64),
        ("trips", ctypes.c_int64),
        ("resident_grid", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["variant_name"] = VARIANT_NAMES.get(self.variant, str(self.variant))
        return d

    def copy(self, **changes) -> "Plan":
        p = Plan()
        ctypes.pointer(p)[0] = self
        for k, v in changes.items():
            setattr(p, k, v)
        return p


class Layout(ctypes.Structure):
    """rmsnorm_layout_t: rows per batch (0 = one batch) and element strides of x and y."""
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("x_row_stride", ctypes.c_int64),
        ("x_batch_stride", ctypes.c_int64),
        ("y_row_stride", ctypes.c_int64),
        ("y_batch_stride", ctypes.c_int64),
    ]


class BwdLayout(ctypes.Structure):
    """rmsnorm_bwd_layout_t: rows per batch (0 = one batch) and element strides of x, dy and dx."""
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("x_row_stride", ctypes.c_int64),
        ("x_batch_stride", ctypes.c_int64),
        ("dy_row_stride", ctypes.c_int64),
        ("dy_batch_stride", ctypes.c_int64),
        ("dx_row_stride", ctypes.c_int64),
        ("dx_batch_stride", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIBRARY):
        raise ImportError(
            f"{LIBRARY} is not built; run `python -m memory_bound_row_rmsnorm_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIBRARY)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.rmsnorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, f32, i32, vp]
    lib.rmsnorm_fwd.restype = i32
    lib.rmsnorm_fwd_with_plan.argtypes = [vp, vp, vp, vp, i64, i64, f32, f32, i32,
                                          ctypes.POINTER(Plan), vp]
    lib.rmsnorm_fwd_with_plan.restype = i32
    lib.rmsnorm_plan_query.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.c_int32, ctypes.POINTER(Plan)]
    lib.rmsnorm_plan_query.restype = i32
    lib.rmsnorm_fwd_ex.argtypes = [vp, vp, vp, vp, i64, i64, f32, f32, i32, ctypes.POINTER(Layout),
                                   ctypes.POINTER(Plan), vp]
    lib.rmsnorm_fwd_ex.restype = i32
    lib.rmsnorm_plan_query_ex.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.POINTER(Layout), ctypes.c_int32,
                                          ctypes.POINTER(Plan)]
    lib.rmsnorm_plan_query_ex.restype = i32
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.rmsnorm_plan_resources.argtypes = [ctypes.POINTER(Plan), i32, i32p, i32p, i32p, i32p]
    lib.rmsnorm_plan_resources.restype = i32
    lib.rmsnorm_fwd_kernel_query.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.POINTER(Plan),
                                             ctypes.POINTER(ctypes.c_char_p), i32p, i32p, i32p]
    lib.rmsnorm_fwd_kernel_query.restype = i32
    lib.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp, i64, vp]
    lib.rmsnorm_bwd.restype = i32
    lib.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
    lib.rmsnorm_bwd_noalloc.restype = i32
    lib.rmsnorm_bwd_with_plan.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32,
                                          ctypes.POINTER(Plan), vp, i64, vp]
    lib.rmsnorm_bwd_with_plan.restype = i32
    lib.rmsnorm_bwd_plan_query.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.c_int32, ctypes.POINTER(Plan)]
    lib.rmsnorm_bwd_plan_query.restype = i32
    lib.rmsnorm_bwd_workspace_size.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_int64)]
    lib.rmsnorm_bwd_workspace_size.restype = i32
    lib.rmsnorm_bwd_plan_validate.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.POINTER(Plan), ctypes.c_int32,
                                              ctypes.POINTER(Plan)]
    lib.rmsnorm_bwd_plan_validate.restype = i32
    lib.rmsnorm_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, ctypes.POINTER(BwdLayout),
                                   ctypes.POINTER(Plan), vp, i64, vp]
    lib.rmsnorm_bwd_ex.restype = i32
    lib.rmsnorm_bwd_plan_query_ex.argtypes = [i64, i64, i32, vp, vp, vp, vp, ctypes.POINTER(BwdLayout),
                                              ctypes.c_int32, ctypes.POINTER(Plan)]
    lib.rmsnorm_bwd_plan_query_ex.restype = i32
    lib.rmsnorm_bwd_workspace_size_ex.argtypes = [i64, i64, i32, vp, vp, vp, vp, ctypes.POINTER(BwdLayout),
                                                  ctypes.POINTER(ctypes.c_int64)]
    lib.rmsnorm_bwd_workspace_size_ex.restype = i32
    lib.rmsnorm_plan_validate.argtypes = [i64, i64, i32, vp, vp, vp, ctypes.POINTER(Plan), ctypes.c_int32,
                                          ctypes.POINTER(Plan)]
    lib.rmsnorm_plan_validate.restype = i32
    lib.rmsnorm_plan_set_tuned.argtypes = [i64, i64, i32, ctypes.POINTER(Plan)]
    lib.rmsnorm_plan_set_tuned.restype = i32
    lib.rmsnorm_plan_clear_tuned.argtypes = []
    lib.rmsnorm_plan_clear_tuned.restype = i32
    lib.rmsnorm_plan_tuned_count.argtypes = []
    lib.rmsnorm_plan_tuned_count.restype = i32
    lib.rmsnorm_status_string.argtypes = [i32]
    lib.rmsnorm_status_string.restype = ctypes.c_char_p
    lib.rmsnorm_last_error.argtypes = []
    lib.rmsnorm_last_error.restype = ctypes.c_char_p
    lib.rmsnorm_version.argtypes = []
    lib.rmsnorm_version.restype = i32
    return lib


lib = _load()


def library_path() -> str:
    return LIBRARY


def status_string(status: int) -> str:
    return lib.rmsnorm_status_string(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise RmsnormError(status, lib.rmsnorm_last_error().decode())


def _dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        if dtype not in DTYPE_NAMES:
            raise ValueError(f"dtype must be 'bf16', 'fp16' or 'fp32', got {dtype!r}")
        return DTYPE_NAMES[dtype]
    if dtype not in DTYPE_CODES:
        raise ValueError(f"dtype must be torch.bfloat16, torch.float16 or torch.float32, got {dtype}")
    return DTYPE_CODES[dtype]


def _stream_handle(stream) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream or None


def _check_tensors(x: torch.Tensor, w: torch.Tensor):
    if not (x.is_cuda and w.is_cuda):
        raise ValueError("x and w must be GPU tensors")
    if x.device != w.device:
        raise ValueError(f"x on {x.device} but w on {w.device}")
    if x.dtype != w.dtype:
        raise ValueError(f"x is {x.dtype} but w is {w.dtype}; both must have the same dtype")
    _dtype_code(x.dtype)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [M, N], got shape {tuple(x.shape)}")
    if w.dim() != 1 or w.shape[0] != x.shape[1]:
        raise ValueError(f"w must have shape [{x.shape[1]}], got {tuple(w.shape)}")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous (no implicit copies are made)")


def rmsnorm_fwd_out(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, rstd: torch.Tensor,
                    eps: float = 1e-6, offset: float = 0.0, plan: Plan | None = None,
                    stream=None) -> None:
    """Write y (x's dtype, [M, N]) and rstd (fp32, [M]) in place; enqueue only."""
    _check_tensors(x, w)
    M, N = x.shape
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous() or y.device != x.device:
        raise ValueError("y must be a contiguous tensor like x")
    if (rstd.shape != (M,) or rstd.dtype != torch.float32 or not rstd.is_contiguous()
            or rstd.device != x.device):
        raise ValueError(f"rstd must be a contiguous float32 tensor of shape [{M}] on {x.device}")
    args = (x.data_ptr(), w.data_ptr(), y.data_ptr(), rstd.data_ptr(), M, N, eps, offset,
            DTYPE_CODES[x.dtype])
    with torch.cuda.device(x.device):
        h = _stream_handle(stream)
        if plan is None:
            _check(lib.rmsnorm_fwd(*args, h))
        else:
            _check(lib.rmsnorm_fwd_with_plan(*args, ctypes.byref(plan), h))


def row_layout(t: torch.Tensor):
    """(M, N, rows, row_stride, batch_stride) of the rows of `t` over its last dimension.

    The last dimension must have unit stride.  A 1-D or 2-D tensor is one batch of rows
    (rows = 0) with t.stride(0) between rows; a tensor of higher rank is batches of
    t.shape[-2] rows, its leading dimensions collapsing into one batch stride (raises
    ValueError when they do not).
    """
    if t.dim() == 0:
        raise ValueError("a 0-d tensor has no rows")
    N = t.shape[-1]
    if N > 1 and t.stride(-1) != 1:
        raise ValueError("the last dimension must have unit stride")
    if t.dim() == 1:
        return 1, N, 0, N, 0
    if t.dim() == 2:
        return t.shape[0], N, 0, t.stride(0), 0
    S, rs = t.shape[-2], t.stride(-2)
    lead = [(n, st) for n, st in zip(t.shape[:-2], t.stride()[:-2]) if n != 1]
    B = 1
    for n, _ in lead:
        B *= n
    bs = lead[-1][1] if lead else 0
    for (n0, s0), (n1, s1) in zip(lead, lead[1:]):
        if s0 != s1 * n1:
            raise ValueError(f"leading dimensions {tuple(t.shape[:-2])} with strides {tuple(t.stride()[:-2])} "
                             "do not collapse into one batch stride")
    return B * S, N, S, rs, bs


def rmsnorm_fwd_ex(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, offset: float = 0.0,
                   want_rstd: bool = True, out: torch.Tensor | None = None, plan: Plan | None = None,
                   stream=None):
    """RMSNorm over the last dimension of x of any rank and strides (unit stride in the last
    dimension), without copies: (y, rstd) with y shaped like x (or written into `out`) and rstd
    float32 of shape x.shape[:-1], or None when want_rstd is False.  bf16, fp16 or fp32."""
    if not (x.is_cuda and w.is_cuda) or x.device != w.device:
        raise ValueError("x and w must be tensors on the same GPU")
    if x.dtype != w.dtype:
        raise ValueError(f"x is {x.dtype} but w is {w.dtype}; both must have the same dtype")
    code = _dtype_code(x.dtype)
    if w.dim() != 1 or w.shape[0] != x.shape[-1] or not w.is_contiguous():
        raise ValueError(f"w must be contiguous with shape [{x.shape[-1]}], got {tuple(w.shape)}")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or y.device != x.device:
        raise ValueError("out must have x's shape, dtype and device")
    M, N, rows, xrs, xbs = row_layout(x)
    _, _, yrows, yrs, ybs = row_layout(y)
    if x.dim() >= 3 and rows != yrows:
        raise ValueError("x and out batch their rows differently")
    lay = Layout(rows, xrs, xbs, yrs, ybs)
    rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if want_rstd else None
    with torch.cuda.device(x.device):
        _check(lib.rmsnorm_fwd_ex(x.data_ptr() or None, w.data_ptr() or None, y.data_ptr() or None,
                                  rstd.data_ptr() if rstd is not None and rstd.numel() else None, M, N, eps,
                                  offset, code, ctypes.byref(lay), ctypes.byref(plan) if plan is not None else None,
                                  _stream_handle(stream)))
    return y, rstd


def plan_query_ex(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None, cu_count: int = 0) -> Plan:
    """The plan rmsnorm_fwd_ex uses for these tensors (one batch of rows)."""
    y = x if out is None else out
    M, N, rows, xrs, xbs = row_layout(x)
    _, _, _, yrs, ybs = row_layout(y)
    p = Plan()
    _check(lib.rmsnorm_plan_query_ex(M, N, _dtype_code(x.dtype), x.data_ptr() or None, w.data_ptr() or None,
                                     y.data_ptr() or None, ctypes.byref(Layout(rows, xrs, xbs, yrs, ybs)),
                                     cu_count, ctypes.byref(p)))
    return p


def rmsnorm_fwd(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, offset: float = 0.0,
                plan: Plan | None = None, stream=None):
    """y = x * rsqrt(mean(x^2, -1) + eps) * (offset + w) and rstd, on x's GPU.

    Returns (y, rstd) with y of x's dtype and rstd float32 [M].
    """
    _check_tensors(x, w)
    y = torch.empty_like(x)
    rstd = torch.empty((x.shape[0],), dtype=torch.float32, device=x.device)
    rmsnorm_fwd_out(x, w, y, rstd, eps, offset, plan, stream)
    return y, rstd


def plan_query(M: int, N: int, dtype, x_ptr: int = 0, w_ptr: int = 0, y_ptr: int = 0,
               cu_count: int = 0) -> Plan:
    """The plan rmsnorm_fwd uses; cu_count > 0 sizes resident_grid without a GPU."""
    p = Plan()
    _check(lib.rmsnorm_plan_query(M, N, _dtype_code(dtype), x_ptr or None, w_ptr or None,
                                  y_ptr or None, cu_count, ctypes.byref(p)))
    return p


def plan_resources(plan: Plan, dtype) -> dict:
    """VGPRs, LDS bytes and scratch bytes of the kernel a plan selects (needs a GPU)."""
    v, s, l, sc = (ctypes.c_int32() for _ in range(4))
    _check(lib.rmsnorm_plan_resources(ctypes.byref(plan), _dtype_code(dtype), ctypes.byref(v),
                                      ctypes.byref(s), ctypes.byref(l), ctypes.byref(sc)))
    return {"vgprs": v.value, "lds_bytes": l.value, "scratch_bytes": sc.value}


def kernel_query(M: int, N: int, dtype, x_ptr: int = 0, w_ptr: int = 0, y_ptr: int = 0,
                 plan: Plan | None = None, resources: bool = True) -> dict:
    """The kernel instance a forward launch over contiguous [M, N] rows with these pointers and
    plan (None = the library's) runs, and (``resources``, needs a GPU) its VGPRs, LDS bytes and
    scratch bytes."""
    name = ctypes.c_char_p()
    v, l, sc = (ctypes.c_int32() for _ in range(3))
    refs = (ctypes.byref(v), ctypes.byref(l), ctypes.byref(sc)) if resources else (None, None, None)
    _check(lib.rmsnorm_fwd_kernel_query(M, N, _dtype_code(dtype), x_ptr or None, w_ptr or None, y_ptr or None,
                                        ctypes.byref(plan) if plan is not None else None, ctypes.byref(name),
                                        *refs))
    out = {"kernel": name.value.decode()}
    if resources:
        out.update({"vgprs": v.value, "lds_bytes": l.value, "scratch_bytes": sc.value})
    return out


def version() -> int:
    return lib.rmsnorm_version()


# ---------------------------------------------------------------------------
# Tuned dispatch
# ---------------------------------------------------------------------------
PLAN_FIELDS = ("variant", "lanes_per_row", "vectors_per_lane", "row_slots", "block_threads", "prefetch",
               "xcd_group", "max_blocks_per_cu", "grid")


def plan_validate(M: int, N: int, dtype, plan: Plan, x_ptr: int = 0, w_ptr: int = 0, y_ptr: int = 0,
                  cu_count: int = 0):
    """The completed plan (derived fields, resident_grid), or None if rmsnorm_fwd_with_plan would
    reject it for these sizes and pointers.  Other errors raise."""
    out = Plan()
    st = lib.rmsnorm_plan_validate(M, N, _dtype_code(dtype), x_ptr or None, w_ptr or None, y_ptr or None,
                                   ctypes.byref(plan), cu_count, ctypes.byref(out))
    if st == 8:
        return None
    _check(st)
    return out


def set_tuned(M: int, N: int, dtype, plan: Plan) -> None:
    """Register `plan` for forward calls of exactly this shape and dtype."""
    _check(lib.rmsnorm_plan_set_tuned(M, N, _dtype_code(dtype), ctypes.byref(plan)))


def clear_tuned() -> None:
    _check(lib.rmsnorm_plan_clear_tuned())


def tuned_count() -> int:
    return lib.rmsnorm_plan_tuned_count()


def load_tuned(path: str) -> int:
    """Register every plan of a tuning file (JSON: {"plans": [{"M", "N", "dtype", "plan": {...}}]});
    returns how many were registered."""
    import json

    with open(path) as f:
        doc = json.load(f)
    n = 0
    for e in doc["plans"]:
        p = Plan()
        for k in PLAN_FIELDS:
            setattr(p, k, int(e["plan"][k]))
        set_tuned(int(e["M"]), int(e["N"]), e["dtype"], p)
        n += 1
    return n


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def bwd_plan_query(M: int, N: int, dtype, x_ptr: int = 0, dy_ptr: int = 0, dx_ptr: int = 0,
                   cu_count: int = 0) -> Plan:
    """The row-pass plan rmsnorm_bwd uses (grid = number of dw partial rows)."""
    p = Plan()
    _check(lib.rmsnorm_bwd_plan_query(M, N, _dtype_code(dtype), x_ptr or None, dy_ptr or None,
                                      dx_ptr or None, cu_count, ctypes.byref(p)))
    return p


def bwd_plan_validate(M: int, N: int, dtype, plan: Plan, x_ptr: int = 0, dy_ptr: int = 0, dx_ptr: int = 0,
                      cu_count: int = 0):
    """The completed backward plan (derived fields, resident_grid), or None if
    rmsnorm_bwd_with_plan would reject it for these sizes and pointers.  Other errors raise."""
    out = Plan()
    st = lib.rmsnorm_bwd_plan_validate(M, N, _dtype_code(dtype), x_ptr or None, dy_ptr or None, dx_ptr or None,
                                       ctypes.byref(plan), cu_count, ctypes.byref(out))
    if st == 8:
        return None
    _check(st)
    return out


def bwd_workspace_size(M: int, N: int, dtype, x_ptr: int = 0, dy_ptr: int = 0, dx_ptr: int = 0) -> int:
    b = ctypes.c_int64()
    _check(lib.rmsnorm_bwd_workspace_size(M, N, _dtype_code(dtype), x_ptr or None, dy_ptr or None,
                                          dx_ptr or None, ctypes.byref(b)))
    return b.value


def rmsnorm_bwd_out(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rstd: torch.Tensor,
                    dx: torch.Tensor, dw: torch.Tensor, workspace: torch.Tensor, offset: float = 0.0,
                    plan: Plan | None = None, stream=None) -> None:
    """Write dx (x's dtype) and dw (fp32 [N]); workspace is any device tensor
    of at least the required bytes.  Enqueue only."""
    _check_tensors(x, w)
    M, N = x.shape
    for name, t in (("dy", dy), ("dx", dx)):
        if t.shape != x.shape or t.dtype != x.dtype or not t.is_contiguous() or t.device != x.device:
            raise ValueError(f"{name} must be a contiguous tensor like x")
    if rstd.shape != (M,) or rstd.dtype != torch.float32 or not rstd.is_contiguous() or rstd.device != x.device:
        raise ValueError(f"rstd must be a contiguous float32 tensor of shape [{M}] on {x.device}")
    if dw.shape != (N,) or dw.dtype != torch.float32 or not dw.is_contiguous() or dw.device != x.device:
        raise ValueError(f"dw must be a contiguous float32 tensor of shape [{N}] on {x.device}")
    if not workspace.is_contiguous() or workspace.device != x.device:
        raise ValueError("workspace must be a contiguous tensor on x's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (x.data_ptr(), w.data_ptr(), dy.data_ptr(), rstd.data_ptr(), dx.data_ptr(), dw.data_ptr(),
            M, N, offset, DTYPE_CODES[x.dtype])
    with torch.cuda.device(x.device):
        h = _stream_handle(stream)
        if plan is None:
            _check(lib.rmsnorm_bwd(*args, workspace.data_ptr() or None, ws_bytes, h))
        else:
            _check(lib.rmsnorm_bwd_with_plan(*args, ctypes.byref(plan), workspace.data_ptr() or None,
                                             ws_bytes, h))


def rmsnorm_bwd(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rstd: torch.Tensor,
                offset: float = 0.0, plan: Plan | None = None, stream=None):
    """Gradients of y = x * rstd * (offset + w) given dy and the forward's rstd.

    Returns (dx of x's dtype, dw float32 [N]).
    """
    _check_tensors(x, w)
    M, N = x.shape
    dx = torch.empty_like(x)
    dw = torch.empty((N,), dtype=torch.float32, device=x.device)
    if plan is None:
        b = ctypes.c_int64()
        _check(lib.rmsnorm_bwd_workspace_size_ex(M, N, _dtype_code(x.dtype), x.data_ptr() or None,
                                                 w.data_ptr() or None, dy.data_ptr() or None,
                                                 dx.data_ptr() or None, None, ctypes.byref(b)))
        nbytes = b.value
    else:
        nbytes = plan.grid * N * 4 if M > 0 else 0
    ws = torch.empty((max(nbytes, 16) + 3) // 4, dtype=torch.float32, device=x.device)
    rmsnorm_bwd_out(x, w, dy, rstd, dx, dw, ws, offset, plan, stream)
    return dx, dw


def rmsnorm_bwd_noalloc_out(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rstd: torch.Tensor,
                            dx: torch.Tensor, dw: torch.Tensor, offset: float = 0.0, stream=None) -> None:
    """rmsnorm_bwd_noalloc into caller-provided dx and dw: no workspace, nothing allocated (the
    library's per-GPU scratch holds the dw partial rows)."""
    _check_tensors(x, w)
    M, N = x.shape
    for t, name in ((dy, "dy"), (dx, "dx")):
        if t.shape != x.shape or t.dtype != x.dtype or not t.is_contiguous() or t.device != x.device:
            raise ValueError(f"{name} must be a contiguous tensor shaped and typed like x on x's device")
    if rstd.dtype != torch.float32 or rstd.shape != (M,) or not rstd.is_contiguous():
        raise ValueError("rstd must be a contiguous float32 tensor of shape (M,)")
    if dw.dtype != torch.float32 or dw.shape != (N,) or not dw.is_contiguous():
        raise ValueError("dw must be a contiguous float32 tensor of shape (N,)")
    with torch.cuda.device(x.device):      # the scratch of x's device
        _check(lib.rmsnorm_bwd_noalloc(x.data_ptr() or None, w.data_ptr() or None, dy.data_ptr() or None,
                                       rstd.data_ptr() or None, dx.data_ptr() or None, dw.data_ptr(), M, N,
                                       float(offset), _dtype_code(x.dtype), _stream_handle(stream)))


def rmsnorm_bwd_noalloc(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rstd: torch.Tensor,
                        offset: float = 0.0, stream=None):
    """rmsnorm_bwd without a workspace (the library's scratch); returns (dx, dw)."""
    dx = torch.empty_like(x)
    dw = torch.empty((x.shape[1],), dtype=torch.float32, device=x.device)
    rmsnorm_bwd_noalloc_out(x, w, dy, rstd, dx, dw, offset, stream)
    return dx, dw


def bwd_layout(x: torch.Tensor, dy: torch.Tensor, dx: torch.Tensor):
    """(M, N, BwdLayout) of the rows of x, dy and dx (same shape) over their last dimension."""
    if dy.shape != x.shape or dx.shape != x.shape:
        raise ValueError(f"dy {tuple(dy.shape)} and dx {tuple(dx.shape)} must have x's shape {tuple(x.shape)}")
    M, N, rows, xrs, xbs = row_layout(x)
    _, _, _, yrs, ybs = row_layout(dy)
    _, _, _, ors, obs = row_layout(dx)
    return M, N, BwdLayout(rows, xrs, xbs, yrs, ybs, ors, obs)


def rmsnorm_bwd_ex(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, rstd: torch.Tensor, offset: float = 0.0,
                   out: torch.Tensor | None = None, plan: Plan | None = None, stream=None):
    """Backward over the last dimension of x, dy (and dx) of any rank and strides (unit stride in
    the last dimension), without copies: (dx shaped like x, or written into `out`; dw float32
    [N]).  rstd: the forward's float32 rstd, contiguous, x.shape[:-1].  bf16, fp16 or fp32."""
    if not (x.is_cuda and w.is_cuda and dy.is_cuda) or len({x.device, w.device, dy.device}) != 1:
        raise ValueError("x, w and dy must be tensors on the same GPU")
    if not (x.dtype == w.dtype == dy.dtype):
        raise ValueError(f"x, w and dy must share a dtype, got {x.dtype}, {w.dtype}, {dy.dtype}")
    code = _dtype_code(x.dtype)
    if w.dim() != 1 or w.shape[0] != x.shape[-1] or not w.is_contiguous():
        raise ValueError(f"w must be contiguous with shape [{x.shape[-1]}], got {tuple(w.shape)}")
    if rstd.dtype != torch.float32 or not rstd.is_contiguous() or rstd.shape != x.shape[:-1] or \
            rstd.device != x.device:
        raise ValueError(f"rstd must be a contiguous float32 tensor of shape {tuple(x.shape[:-1])} on {x.device}")
    dx = torch.empty_like(x) if out is None else out
    if dx.dtype != x.dtype or dx.device != x.device:
        raise ValueError("out must have x's dtype and device")
    M, N, lay = bwd_layout(x, dy, dx)
    dw = torch.empty((N,), dtype=torch.float32, device=x.device)
    ptrs = (x.data_ptr() or None, w.data_ptr() or None, dy.data_ptr() or None, dx.data_ptr() or None)
    if plan is None:
        b = ctypes.c_int64()
        _check(lib.rmsnorm_bwd_workspace_size_ex(M, N, code, *ptrs, ctypes.byref(lay), ctypes.byref(b)))
        nbytes = b.value
    else:
        nbytes = plan.grid * N * 4 if M > 0 else 0
    ws = torch.empty((max(nbytes, 16) + 3) // 4, dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib.rmsnorm_bwd_ex(x.data_ptr() or None, w.data_ptr() or None, dy.data_ptr() or None,
                                  rstd.data_ptr() or None, dx.data_ptr() or None, dw.data_ptr(), M, N, offset, code,
                                  ctypes.byref(lay), ctypes.byref(plan) if plan is not None else None,
                                  ws.data_ptr(), ws.numel() * 4, _stream_handle(stream)))
    return dx, dw


def bwd_plan_query_ex(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, out: torch.Tensor | None = None,
                      cu_count: int = 0) -> Plan:
    """The row-pass plan rmsnorm_bwd_ex uses for these tensors."""
    dx = x if out is None else out
    M, N, lay = bwd_layout(x, dy, dx)
    p = Plan()
    _check(lib.rmsnorm_bwd_plan_query_ex(M, N, _dtype_code(x.dtype), x.data_ptr() or None, w.data_ptr() or None,
                                         dy.data_ptr() or None, dx.data_ptr() or None, ctypes.byref(lay), cu_count,
                                         ctypes.byref(p)))
    return p
