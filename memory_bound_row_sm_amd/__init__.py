"""Python binding of the gfx950 row-softmax library (``libsm_softmax.so``).

Argument marshalling only: every function calls the C entry point of the same
name declared in ``include/sm_softmax.h`` / ``include/sm_bench.h``; all work runs
in the library's HIP kernels. PyTorch is used for device memory and streams in
``softmax()``, a convenience wrapper that passes a tensor's pointer, row stride
and the current stream to ``sm_softmax_fwd_ex``.

There is no fallback: if the library is not built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SM_F32", "SM_F16", "SM_BF16", "SM_PLAN_AUTO", "SM_PLAN_RESIDENT", "SM_PLAN_PERSISTENT",
    "SM_PLAN_WIDE", "SM_PLAN_SPLIT", "SmOpts", "SmPlanInfo", "SoftmaxError", "lib", "lib_path",
    "sm_softmax_fwd", "sm_softmax_fwd_ex", "sm_softmax_plan_query", "sm_softmax_strerror",
    "sm_softmax_version", "sm_softmax_last_hip_error", "sm_bench_copy", "sm_bench_flush",
    "softmax", "plan_for", "EXPORTED_SYMBOLS", "sm_softmax_bwd", "sm_softmax_bwd_ex",
    "sm_softmax_bwd_plan_query", "softmax_backward", "plan_for_backward",
    "sm_softmax_sync_failures", "sync_failures", "sm_rmsnorm_fwd", "sm_rmsnorm_fwd_ex",
    "sm_rmsnorm_plan_query", "rmsnorm", "plan_for_rmsnorm", "sm_attention_fwd",
    "sm_attention_fwd_ex", "attention", "sm_softmax_fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
]

SM_F32, SM_F16, SM_BF16 = 0, 1, 2
SM_PLAN_AUTO, SM_PLAN_RESIDENT, SM_PLAN_PERSISTENT, SM_PLAN_WIDE, SM_PLAN_SPLIT = 0, 1, 2, 3, 4
PLAN_NAMES = {SM_PLAN_AUTO: "auto", SM_PLAN_RESIDENT: "resident",
              SM_PLAN_PERSISTENT: "persistent", SM_PLAN_WIDE: "wide", SM_PLAN_SPLIT: "split"}
STATUS = {0: "SM_OK", -1: "SM_ERR_INVALID", -2: "SM_ERR_DTYPE", -3: "SM_ERR_OVERLAP",
          -4: "SM_ERR_HIP", -5: "SM_ERR_NO_DEVICE", -6: "SM_ERR_WORKSPACE", -7: "SM_ERR_PLAN"}

EXPORTED_SYMBOLS = (
    "sm_softmax_fwd", "sm_softmax_fwd_ex", "sm_softmax_plan_query", "sm_softmax_bwd",
    "sm_softmax_bwd_ex", "sm_softmax_bwd_plan_query", "sm_softmax_strerror",
    "sm_softmax_version", "sm_softmax_last_hip_error", "sm_softmax_sync_failures",
    "sm_rmsnorm_fwd", "sm_rmsnorm_fwd_ex", "sm_rmsnorm_plan_query",
    "sm_attention_fwd", "sm_attention_fwd_ex", "sm_bench_copy", "sm_bench_flush",
    "sm_softmax_fwd_noalloc",
)
NOALLOC_SCRATCH_BYTES = 1 << 20  # SM_NOALLOC_SCRATCH_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libsm_softmax.so")
ABI_VERSION = 10200  # SM_SOFTMAX_VERSION of the signatures declared below


class SmOpts(ctypes.Structure):
    _fields_ = [("plan", ctypes.c_int), ("lanes_per_row", ctypes.c_int),
                ("vecs_per_lane", ctypes.c_int), ("grid", ctypes.c_int),
                ("chunks_per_wave", ctypes.c_int), ("prefetch", ctypes.c_int),
                ("nontemporal", ctypes.c_int), ("spin_limit", ctypes.c_int),
                ("start_event", ctypes.c_void_p), ("stop_event", ctypes.c_void_p)]


class SmPlanInfo(ctypes.Structure):
    _fields_ = [("plan", ctypes.c_int), ("lanes_per_row", ctypes.c_int),
                ("vecs_per_lane", ctypes.c_int), ("prefetch", ctypes.c_int),
                ("nt_loads", ctypes.c_int), ("block", ctypes.c_int), ("grid", ctypes.c_int64),
                ("chunks_per_wave", ctypes.c_int), ("waves_per_row", ctypes.c_int64),
                ("launches", ctypes.c_int), ("same_phase", ctypes.c_int),
                ("workspace_bytes", ctypes.c_int64), ("model_bytes", ctypes.c_int64),
                ("dy_same_phase", ctypes.c_int), ("slice_windows", ctypes.c_int)]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["plan_name"] = PLAN_NAMES.get(self.plan, str(self.plan))
        return d


class SoftmaxError(RuntimeError):
    def __init__(self, status: int, where: str = "sm_softmax"):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({sm_softmax_strerror(status)})"
        if status == -4:
            msg += f", hipError {sm_softmax_last_hip_error()}"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        try:
            # torch ships its own copy of the HIP runtime under the same soname; loading
            # torch first makes this library bind to that copy, so torch's device pointers
            # and stream handles belong to the runtime our kernels are launched through
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(lib_path):
            raise RuntimeError(
                f"{lib_path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python memory_bound_row_sm_amd/build.py`")
        L = ctypes.CDLL(lib_path)
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.sm_softmax_fwd.argtypes = [vp, vp, i64, i64, i64, i64, ci, vp]
        L.sm_softmax_fwd_noalloc.argtypes = [vp, vp, i64, i64, i64, i64, ci, vp]
        L.sm_softmax_fwd_ex.argtypes = [vp, vp, i64, i64, i64, i64, ci, ctypes.POINTER(SmOpts),
                                        vp, ctypes.c_size_t, vp]
        L.sm_softmax_plan_query.argtypes = [vp, vp, i64, i64, i64, i64, ci,
                                            ctypes.POINTER(SmOpts), ci, ctypes.POINTER(SmPlanInfo)]
        L.sm_softmax_bwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ci, vp]
        L.sm_softmax_bwd_ex.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ci,
                                        ctypes.POINTER(SmOpts), vp, ctypes.c_size_t, vp]
        L.sm_softmax_bwd_plan_query.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ci,
                                                ctypes.POINTER(SmOpts), ci,
                                                ctypes.POINTER(SmPlanInfo)]
        cf = ctypes.c_float
        L.sm_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, cf, ci, vp]
        L.sm_rmsnorm_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, cf, ci,
                                        ctypes.POINTER(SmOpts), vp, ctypes.c_size_t, vp]
        L.sm_rmsnorm_plan_query.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, cf,
                                            ci, ctypes.POINTER(SmOpts), ci,
                                            ctypes.POINTER(SmPlanInfo)]
        attn = [vp, vp, vp, vp, vp] + [i64] * 12 + [cf, ci, ci]
        L.sm_attention_fwd.argtypes = attn + [vp]
        L.sm_attention_fwd_ex.argtypes = attn + [ctypes.POINTER(SmOpts), vp]
        L.sm_softmax_strerror.argtypes = [ci]
        L.sm_softmax_strerror.restype = ctypes.c_char_p
        L.sm_softmax_version.argtypes = []
        L.sm_softmax_last_hip_error.argtypes = []
        L.sm_softmax_sync_failures.argtypes = [vp, ctypes.POINTER(ctypes.c_uint)]
        L.sm_bench_copy.argtypes = [vp, vp, ctypes.c_size_t, ci, ci, vp, vp, vp]
        L.sm_bench_flush.argtypes = [vp, ctypes.c_size_t, vp]
        for f in (L.sm_softmax_fwd, L.sm_softmax_fwd_noalloc, L.sm_softmax_fwd_ex,
                  L.sm_softmax_plan_query,
                  L.sm_softmax_bwd, L.sm_softmax_bwd_ex, L.sm_softmax_bwd_plan_query,
                  L.sm_softmax_version, L.sm_softmax_last_hip_error, L.sm_softmax_sync_failures,
                  L.sm_rmsnorm_fwd, L.sm_rmsnorm_fwd_ex, L.sm_rmsnorm_plan_query,
                  L.sm_attention_fwd, L.sm_attention_fwd_ex, L.sm_bench_copy, L.sm_bench_flush):
            f.restype = ci
        if L.sm_softmax_version() != ABI_VERSION:
            raise RuntimeError(
                f"{lib_path} reports version {L.sm_softmax_version()}, the binding expects "
                f"{ABI_VERSION}: rebuild with `python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = L
    return _lib


def _opts(opts) -> SmOpts | None:
    if opts is None:
        return None
    if isinstance(opts, SmOpts):
        return opts
    o = SmOpts()  # all zero: automatic
    for k, v in dict(opts).items():
        setattr(o, k, v if k.endswith("_event") else int(v))
    return o


# ---------------------------------------------------------------- C entry points

def sm_softmax_fwd(in_ptr: int, out_ptr: int, M: int, N: int, in_stride: int, out_stride: int,
                   dtype: int, stream: int = 0) -> int:
    return lib().sm_softmax_fwd(in_ptr, out_ptr, M, N, in_stride, out_stride, dtype, stream)


def sm_softmax_fwd_noalloc(in_ptr: int, out_ptr: int, M: int, N: int, in_stride: int,
                           out_stride: int, dtype: int, stream: int = 0) -> int:
    return lib().sm_softmax_fwd_noalloc(in_ptr, out_ptr, M, N, in_stride, out_stride, dtype, stream)


def sm_softmax_fwd_ex(in_ptr: int, out_ptr: int, M: int, N: int, in_stride: int, out_stride: int,
                      dtype: int, opts=None, workspace: int = 0, workspace_bytes: int = 0,
                      stream: int = 0) -> int:
    o = _opts(opts)
    return lib().sm_softmax_fwd_ex(in_ptr, out_ptr, M, N, in_stride, out_stride, dtype,
                                   ctypes.byref(o) if o is not None else None,
                                   workspace or None, workspace_bytes, stream)


def sm_softmax_plan_query(in_ptr: int, out_ptr: int, M: int, N: int, in_stride: int,
                          out_stride: int, dtype: int, opts=None, num_cus: int = 0):
    """(status, SmPlanInfo)."""
    o = _opts(opts)
    info = SmPlanInfo()
    rc = lib().sm_softmax_plan_query(in_ptr, out_ptr, M, N, in_stride, out_stride, dtype,
                                     ctypes.byref(o) if o is not None else None, num_cus,
                                     ctypes.byref(info))
    return rc, info


def sm_softmax_bwd(y_ptr: int, dy_ptr: int, dx_ptr: int, M: int, N: int, y_stride: int,
                   dy_stride: int, dx_stride: int, dtype: int, stream: int = 0) -> int:
    return lib().sm_softmax_bwd(y_ptr, dy_ptr, dx_ptr, M, N, y_stride, dy_stride, dx_stride,
                                dtype, stream)


def sm_softmax_bwd_ex(y_ptr: int, dy_ptr: int, dx_ptr: int, M: int, N: int, y_stride: int,
                      dy_stride: int, dx_stride: int, dtype: int, opts=None, workspace: int = 0,
                      workspace_bytes: int = 0, stream: int = 0) -> int:
    o = _opts(opts)
    return lib().sm_softmax_bwd_ex(y_ptr, dy_ptr, dx_ptr, M, N, y_stride, dy_stride, dx_stride,
                                   dtype, ctypes.byref(o) if o is not None else None,
                                   workspace or None, workspace_bytes, stream)


def sm_softmax_bwd_plan_query(y_ptr: int, dy_ptr: int, dx_ptr: int, M: int, N: int,
                              y_stride: int, dy_stride: int, dx_stride: int, dtype: int,
                              opts=None, num_cus: int = 0):
    """(status, SmPlanInfo)."""
    o = _opts(opts)
    info = SmPlanInfo()
    rc = lib().sm_softmax_bwd_plan_query(y_ptr, dy_ptr, dx_ptr, M, N, y_stride, dy_stride,
                                         dx_stride, dtype,
                                         ctypes.byref(o) if o is not None else None, num_cus,
                                         ctypes.byref(info))
    return rc, info


def sm_rmsnorm_fwd(x_ptr: int, r_ptr: int, w_ptr: int, y_ptr: int, s_ptr: int, M: int, N: int,
                   x_stride: int, r_stride: int, y_stride: int, s_stride: int, eps: float,
                   dtype: int, stream: int = 0) -> int:
    return lib().sm_rmsnorm_fwd(x_ptr, r_ptr or None, w_ptr, y_ptr, s_ptr or None, M, N, x_stride,
                                r_stride, y_stride, s_stride, eps, dtype, stream)


def sm_rmsnorm_fwd_ex(x_ptr: int, r_ptr: int, w_ptr: int, y_ptr: int, s_ptr: int, M: int, N: int,
                      x_stride: int, r_stride: int, y_stride: int, s_stride: int, eps: float,
                      dtype: int, opts=None, workspace: int = 0, workspace_bytes: int = 0,
                      stream: int = 0) -> int:
    o = _opts(opts)
    return lib().sm_rmsnorm_fwd_ex(x_ptr, r_ptr or None, w_ptr, y_ptr, s_ptr or None, M, N,
                                   x_stride, r_stride, y_stride, s_stride, eps, dtype,
                                   ctypes.byref(o) if o is not None else None,
                                   workspace or None, workspace_bytes, stream)


def sm_rmsnorm_plan_query(x_ptr: int, r_ptr: int, w_ptr: int, y_ptr: int, s_ptr: int, M: int,
                          N: int, x_stride: int, r_stride: int, y_stride: int, s_stride: int,
                          eps: float, dtype: int, opts=None, num_cus: int = 0):
    o = _opts(opts)
    info = SmPlanInfo()
    rc = lib().sm_rmsnorm_plan_query(x_ptr, r_ptr or None, w_ptr, y_ptr, s_ptr or None, M, N,
                                     x_stride, r_stride, y_stride, s_stride, eps, dtype,
                                     ctypes.byref(o) if o is not None else None, num_cus,
                                     ctypes.byref(info))
    return rc, info


def sm_attention_fwd(q: int, k: int, v: int, o: int, lse: int, BH: int, Sq: int, Sk: int, d: int,
                     strides, scale: float, causal: int, dtype: int, stream: int = 0) -> int:
    """``strides``: (q_row, q_head, k_row, k_head, v_row, v_head, o_row, o_head) in elements."""
    return lib().sm_attention_fwd(q, k or None, v or None, o, lse or None, BH, Sq, Sk, d, *strides,
                                  scale, causal, dtype, stream)


def sm_attention_fwd_ex(q: int, k: int, v: int, o: int, lse: int, BH: int, Sq: int, Sk: int, d: int,
                        strides, scale: float, causal: int, dtype: int, opts=None,
                        stream: int = 0) -> int:
    oo = _opts(opts)
    return lib().sm_attention_fwd_ex(q, k or None, v or None, o, lse or None, BH, Sq, Sk, d,
                                     *strides, scale, causal, dtype,
                                     ctypes.byref(oo) if oo is not None else None, stream)


def sm_softmax_strerror(status: int) -> str:
    return lib().sm_softmax_strerror(status).decode()


def sm_softmax_version() -> int:
    return lib().sm_softmax_version()


def sm_softmax_last_hip_error() -> int:
    return lib().sm_softmax_last_hip_error()


def sm_softmax_sync_failures(stream: int = 0) -> tuple[int, int]:
    """(status, count): SPLIT waits that ran out of polls on ``stream``."""
    c = ctypes.c_uint(0)
    rc = lib().sm_softmax_sync_failures(stream, ctypes.byref(c))
    return rc, c.value


def sm_bench_copy(src: int, dst: int, nbytes: int, grid: int = 0, store_scope: int = 0,
                  stream: int = 0, start_event=None, stop_event=None) -> int:
    return lib().sm_bench_copy(src, dst, nbytes, grid, store_scope, stream, start_event, stop_event)


def sm_bench_flush(buf: int, nbytes: int, stream: int = 0) -> int:
    return lib().sm_bench_flush(buf, nbytes, stream)


# ---------------------------------------------------------------- torch marshalling

def _torch_dtype_code(t) -> int:
    import torch
    codes = {torch.float32: SM_F32, torch.float16: SM_F16, torch.bfloat16: SM_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _rows_view(t):
    """(M, N, row_stride) of a tensor softmaxed along its last dimension."""
    if t.dim() == 0:
        raise ValueError("expected at least one dimension")
    if t.stride(-1) != 1 and t.size(-1) > 1:
        raise ValueError("the last dimension must be contiguous")
    N = t.size(-1)
    if t.dim() == 1:
        return 1, N, N
    lead = t.shape[:-1]
    M = 1
    for s in lead:
        M *= s
    # leading dimensions must collapse to one row stride
    stride = t.stride(-2)
    exp = stride
    for d in range(t.dim() - 2, -1, -1):
        if t.size(d) != 1 and t.stride(d) != exp:
            raise ValueError("leading dimensions do not collapse to one row stride")
        exp *= t.size(d)
    return M, N, (stride if M > 1 else N)


def softmax(x, out=None, opts=None, workspace=None, stream=None):
    """Row softmax of a CUDA(HIP) tensor along its last dimension, on the current
    stream (or ``stream``). Returns ``out`` (allocated like ``x`` if None)."""
    import torch
    if not x.is_cuda:
        raise ValueError("softmax expects a device tensor (the library has no CPU path)")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.shape != x.shape or out.dtype != x.dtype or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    M, N, si = _rows_view(x)
    _, _, so = _rows_view(out)
    s = (stream if stream is not None else torch.cuda.current_stream(x.device)).cuda_stream
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        rc = sm_softmax_fwd_ex(x.data_ptr(), out.data_ptr(), M, N, si, so, _torch_dtype_code(x),
                               opts, ws_ptr, ws_bytes, s)
    if rc != 0:
        raise SoftmaxError(rc, "sm_softmax_fwd_ex")
    return out


def plan_for(x, out=None, opts=None, num_cus: int = 0) -> dict:
    """The plan ``softmax(x, out, opts)`` would launch, as a dict."""
    out = x if out is None else out
    M, N, si = _rows_view(x)
    _, _, so = _rows_view(out)
    rc, info = sm_softmax_plan_query(x.data_ptr(), out.data_ptr(), M, N, si, so,
                                     _torch_dtype_code(x), opts, num_cus)
    if rc != 0:
        raise SoftmaxError(rc, "sm_softmax_plan_query")
    return info.as_dict()


def softmax_backward(y, dy, dx=None, opts=None, workspace=None, stream=None):
    """dx = y * (dy - sum(y * dy)) along the last dimension, for device tensors y (the
    softmax output) and dy (the gradient with respect to y). Returns ``dx``."""
    import torch
    if not (y.is_cuda and dy.is_cuda):
        raise ValueError("softmax_backward expects device tensors")
    if y.shape != dy.shape or y.dtype != dy.dtype:
        raise ValueError("y and dy must match in shape and dtype")
    if dx is None:
        dx = torch.empty_like(y, memory_format=torch.contiguous_format)
    M, N, sy = _rows_view(y)
    _, _, sd = _rows_view(dy)
    _, _, sx = _rows_view(dx)
    s = (stream if stream is not None else torch.cuda.current_stream(y.device)).cuda_stream
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(y.device):
        rc = sm_softmax_bwd_ex(y.data_ptr(), dy.data_ptr(), dx.data_ptr(), M, N, sy, sd, sx,
                               _torch_dtype_code(y), opts, ws_ptr, ws_bytes, s)
    if rc != 0:
        raise SoftmaxError(rc, "sm_softmax_bwd_ex")
    return dx


def plan_for_backward(y, dy, dx=None, opts=None, num_cus: int = 0) -> dict:
    dx = y if dx is None else dx
    M, N, sy = _rows_view(y)
    _, _, sd = _rows_view(dy)
    _, _, sx = _rows_view(dx)
    rc, info = sm_softmax_bwd_plan_query(y.data_ptr(), dy.data_ptr(), dx.data_ptr(), M, N, sy, sd,
                                         sx, _torch_dtype_code(y), opts, num_cus)
    if rc != 0:
        raise SoftmaxError(rc, "sm_softmax_bwd_plan_query")
    return info.as_dict()


def sync_failures(stream=None) -> int:
    """SPLIT-plan waits that ran out of polls on ``stream`` (torch's current stream
    by default); synchronises that stream."""
    import torch
    s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    rc, n = sm_softmax_sync_failures(s)
    if rc != 0:
        raise SoftmaxError(rc, "sm_softmax_sync_failures")
    return n


def _rms_args(x, weight, residual, out, residual_out):
    import torch
    if not (x.is_cuda and weight.is_cuda):
        raise ValueError("rmsnorm expects device tensors")
    if weight.dim() != 1 or weight.numel() != x.size(-1) or weight.dtype != x.dtype:
        raise ValueError("weight must be a 1-D tensor of N elements of x's dtype")
    if weight.numel() > 1 and weight.stride(0) != 1:
        raise ValueError("weight must be contiguous")
    for t in (residual, out, residual_out):
        if t is not None and (t.shape != x.shape or t.dtype != x.dtype or t.device != x.device):
            raise ValueError("residual, out and residual_out must match x")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    M, N, sx = _rows_view(x)
    sr = _rows_view(residual)[2] if residual is not None else 0
    sy = _rows_view(out)[2]
    ss = _rows_view(residual_out)[2] if residual_out is not None else 0
    ptr = lambda t: t.data_ptr() if t is not None else 0
    return (x.data_ptr(), ptr(residual), weight.data_ptr(), out.data_ptr(), ptr(residual_out), M, N,
            sx, sr, sy, ss), out


def rmsnorm(x, weight, residual=None, eps: float = 1e-6, out=None, residual_out=None, opts=None,
            workspace=None, stream=None):
    """Fused residual RMSNorm along the last dimension of device tensors:
    s = x + residual (FP32 add, rounded to x's dtype), out = s * weight / rms(s).
    Writes s to ``residual_out`` when given. Returns ``out``."""
    import torch
    args, out = _rms_args(x, weight, residual, out, residual_out)
    s = (stream if stream is not None else torch.cuda.current_stream(x.device)).cuda_stream
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        rc = sm_rmsnorm_fwd_ex(*args, float(eps), _torch_dtype_code(x), opts, ws_ptr, ws_bytes, s)
    if rc != 0:
        raise SoftmaxError(rc, "sm_rmsnorm_fwd_ex")
    return out


def plan_for_rmsnorm(x, weight, residual=None, eps: float = 1e-6, out=None, residual_out=None,
                     opts=None, num_cus: int = 0) -> dict:
    args, out = _rms_args(x, weight, residual, out, residual_out)
    rc, info = sm_rmsnorm_plan_query(*args, float(eps), _torch_dtype_code(x), opts, num_cus)
    if rc != 0:
        raise SoftmaxError(rc, "sm_rmsnorm_plan_query")
    return info.as_dict()


def _heads_view(t):
    """(BH, S, d, row_stride, head_stride) of a [..., S, d] tensor whose leading
    dimensions collapse to one head stride."""
    if t.dim() < 2 or (t.size(-1) > 1 and t.stride(-1) != 1):
        raise ValueError("expected [..., S, d] with a contiguous last dimension")
    S, d = t.size(-2), t.size(-1)
    lead = t.shape[:-2]
    BH = 1
    for n in lead:
        BH *= n
    hs = t.stride(-3) if t.dim() > 2 else S * t.stride(-2)
    exp = hs
    for i in range(t.dim() - 3, -1, -1):
        if t.size(i) != 1 and t.stride(i) != exp:
            raise ValueError("leading dimensions do not collapse to one head stride")
        exp *= t.size(i)
    return BH, S, d, t.stride(-2), hs


def attention(q, k, v, scale=None, causal: bool = False, out=None, lse=None, opts=None,
              stream=None):
    """Fused attention forward of device tensors [..., S, d] (FP16/BF16, d = 64 or 128):
    softmax(scale * q k^T [causal, aligned bottom right]) v. Returns ``out``; fills
    ``lse`` (FP32 [..., Sq]) when given."""
    import math
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("attention expects device tensors")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    BH, Sq, d, qr, qh = _heads_view(q)
    BHk, Sk, dk, kr, kh = _heads_view(k)
    BHv, Sv, dv, vr, vh = _heads_view(v)
    BHo, So, do, orr, oh = _heads_view(out)
    if (BHk, dk) != (BH, d) or (BHv, Sv, dv) != (BH, Sk, d) or (BHo, So, do) != (BH, Sq, d):
        raise ValueError("q, k, v and out shapes do not match")
    if lse is not None and (lse.dtype != torch.float32 or lse.numel() != BH * Sq or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 tensor of BH * Sq elements")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    with torch.cuda.device(q.device):
        rc = sm_attention_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else 0, BH, Sq, Sk, d,
                                 (qr, qh, kr, kh, vr, vh, orr, oh), float(scale), int(bool(causal)),
                                 _torch_dtype_code(q), opts, s)
    if rc != 0:
        raise SoftmaxError(rc, "sm_attention_fwd_ex")
    return out
