"""FP64 row-softmax oracle (forward, backward, fused residual RMSNorm, attention):
a ctypes wrapper over ``liboracle_softmax.so``.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg may import this package. The GPU library and its
Python binding never import it, and the two share no code.

The C source (``oracle_softmax.c``) states the definition it follows and the
readings taken where the pages are silent. Every function here only marshals
numpy buffers into that library.

Arrays: FP32 data is passed as ``numpy.float32``; FP16 and BF16 data are passed
as their raw 16-bit patterns (``numpy.uint16``; ``numpy.float16`` is accepted for
FP16). A 2-D array may be a row-strided view (column stride must be one
element); its row stride is taken from the view.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_softmax.so")

_DP = ctypes.POINTER(ctypes.c_double)


def _code(dtype) -> int:
    if isinstance(dtype, str):
        return DTYPES[dtype]
    return int(dtype)


def _storage(dtype) -> np.dtype:
    return np.dtype(np.float32) if _code(dtype) == F32 else np.dtype(np.uint16)


def _as_storage(a: np.ndarray, dtype) -> np.ndarray:
    a = np.asarray(a)
    want = _storage(dtype)
    if a.dtype == want:
        return a
    if a.dtype.itemsize == want.itemsize and a.dtype.kind in "fiu":
        return a.view(want)
    raise TypeError(f"array of {a.dtype} cannot hold dtype code {_code(dtype)} data")


class Oracle:
    """One loaded copy of the oracle library (``path`` defaults to the built one)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python oracle/build.py` "
                "(or __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_decode.argtypes = [vp, ctypes.c_int, i64, _DP]
        lib.oracle_encode.argtypes = [_DP, ctypes.c_int, i64, vp]
        lib.oracle_softmax_rows.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, _DP, ctypes.c_int]
        lib.oracle_softmax_bwd_rows.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp, i64, _DP,
                                                ctypes.c_int]
        lib.oracle_rmsnorm_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, vp, i64,
                                            ctypes.c_double, _DP, _DP, ctypes.c_int]
        lib.oracle_attention_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                              i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                                              vp, i64, _DP, _DP, ctypes.c_int]
        lib.oracle_max_threads.argtypes = []
        for f in (lib.oracle_decode, lib.oracle_encode, lib.oracle_softmax_rows,
                  lib.oracle_softmax_bwd_rows, lib.oracle_rmsnorm_rows, lib.oracle_attention_rows,
                  lib.oracle_max_threads):
            f.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()

    def decode(self, bits: np.ndarray, dtype) -> np.ndarray:
        """Stored elements -> float64, exactly."""
        src = np.ascontiguousarray(_as_storage(bits, dtype))
        out = np.empty(src.shape, np.float64)
        if self.lib.oracle_decode(src.ctypes.data, _code(dtype), src.size, out.ctypes.data_as(_DP)):
            raise ValueError("oracle_decode rejected its arguments")
        return out

    def encode(self, y: np.ndarray, dtype) -> np.ndarray:
        """float64 -> stored elements, one round-to-nearest-even step."""
        src = np.ascontiguousarray(y, dtype=np.float64)
        out = np.empty(src.shape, _storage(dtype))
        if self.lib.oracle_encode(src.ctypes.data_as(_DP), _code(dtype), src.size, out.ctypes.data):
            raise ValueError("oracle_encode rejected its arguments")
        return out

    def softmax_f64(self, x: np.ndarray, dtype, rows=None, threads: int = 0) -> np.ndarray:
        """FP64 softmax of the rows of a stored 2-D matrix ``x`` (row-strided view allowed).

        ``rows``: optional sequence of row indices; the result then has one row per index.
        """
        a = _as_storage(x, dtype)
        if a.ndim != 2:
            raise ValueError("expected a 2-D matrix")
        es = a.dtype.itemsize
        M, N = a.shape
        nrows = M if rows is None else len(rows)
        if a.size == 0:
            return np.empty((nrows, N), np.float64)
        if N > 1 and a.strides[1] != es:
            raise ValueError("column stride must be one element")
        if a.strides[0] % es or a.strides[0] < 0:
            raise ValueError("row stride must be a non-negative multiple of the element size")
        in_stride = a.strides[0] // es if M > 1 else N
        idx = None
        if rows is not None:
            idx = np.ascontiguousarray(rows, dtype=np.int64)
            if idx.size and (idx.min() < 0 or idx.max() >= M):
                raise IndexError("row index out of range")
        out = np.empty((nrows, N), np.float64)
        rc = self.lib.oracle_softmax_rows(
            a.ctypes.data, _code(dtype), N, in_stride,
            None if idx is None else idx.ctypes.data, nrows, out.ctypes.data_as(_DP), int(threads))
        if rc:
            raise ValueError("oracle_softmax_rows rejected its arguments")
        return out

    def reference(self, x: np.ndarray, dtype, rows=None, threads: int = 0):
        """(y_f64, y_rounded): the FP64 softmax and its one RNE cast to ``dtype``."""
        y = self.softmax_f64(x, dtype, rows=rows, threads=threads)
        return y, self.encode(y, dtype)

    def softmax_bwd_f64(self, y: np.ndarray, dy: np.ndarray, dtype, rows=None,
                        threads: int = 0) -> np.ndarray:
        """FP64 dx = y * (dy - sum(y * dy)) per row, from stored y and dy (2-D, row-strided
        views allowed; same shape and dtype)."""
        a = _as_storage(y, dtype)
        b = _as_storage(dy, dtype)
        if a.ndim != 2 or a.shape != b.shape:
            raise ValueError("y and dy must be 2-D matrices of one shape")
        es = a.dtype.itemsize
        M, N = a.shape
        nrows = M if rows is None else len(rows)
        if a.size == 0:
            return np.empty((nrows, N), np.float64)
        for t in (a, b):
            if N > 1 and t.strides[1] != es:
                raise ValueError("column stride must be one element")
            if t.strides[0] % es or t.strides[0] < 0:
                raise ValueError("row stride must be a non-negative multiple of the element size")
        sa = a.strides[0] // es if M > 1 else N
        sb = b.strides[0] // es if M > 1 else N
        idx = None
        if rows is not None:
            idx = np.ascontiguousarray(rows, dtype=np.int64)
            if idx.size and (idx.min() < 0 or idx.max() >= M):
                raise IndexError("row index out of range")
        out = np.empty((nrows, N), np.float64)
        rc = self.lib.oracle_softmax_bwd_rows(
            a.ctypes.data, b.ctypes.data, _code(dtype), N, sa, sb,
            None if idx is None else idx.ctypes.data, nrows, out.ctypes.data_as(_DP), int(threads))
        if rc:
            raise ValueError("oracle_softmax_bwd_rows rejected its arguments")
        return out

    def reference_bwd(self, y, dy, dtype, rows=None, threads: int = 0):
        """(dx_f64, dx_rounded)."""
        dx = self.softmax_bwd_f64(y, dy, dtype, rows=rows, threads=threads)
        return dx, self.encode(dx, dtype)

    def rmsnorm_f64(self, x: np.ndarray, residual, weight: np.ndarray, dtype, eps: float,
                    rows=None, threads: int = 0):
        """(y_f64, s_f64): residual RMSNorm of the rows of stored x (2-D, row-strided views
        allowed) with an optional stored residual of the same shape and a stored weight of
        N elements; s is the sum rounded once to the dtype (x itself without residual)."""
        a = _as_storage(x, dtype)
        if a.ndim != 2:
            raise ValueError("expected a 2-D matrix")
        M, N = a.shape
        es = a.dtype.itemsize
        b = None if residual is None else _as_storage(residual, dtype)
        if b is not None and b.shape != a.shape:
            raise ValueError("residual must match x")
        w = np.ascontiguousarray(_as_storage(weight, dtype)).reshape(-1)
        if w.size != N:
            raise ValueError("weight must hold N elements")
        nrows = M if rows is None else len(rows)
        y = np.empty((nrows, N), np.float64)
        s = np.empty((nrows, N), np.float64)
        if a.size == 0:
            return y, s
        for t in (a, b) if b is not None else (a,):
            if N > 1 and t.strides[1] != es:
                raise ValueError("column stride must be one element")
            if t.strides[0] % es or t.strides[0] < 0:
                raise ValueError("row stride must be a non-negative multiple of the element size")
        sa = a.strides[0] // es if M > 1 else N
        sb = (b.strides[0] // es if M > 1 else N) if b is not None else 0
        idx = None
        if rows is not None:
            idx = np.ascontiguousarray(rows, dtype=np.int64)
            if idx.size and (idx.min() < 0 or idx.max() >= M):
                raise IndexError("row index out of range")
        rc = self.lib.oracle_rmsnorm_rows(
            a.ctypes.data, None if b is None else b.ctypes.data, w.ctypes.data, _code(dtype), N,
            sa, sb, None if idx is None else idx.ctypes.data, nrows, float(eps),
            y.ctypes.data_as(_DP), s.ctypes.data_as(_DP), int(threads))
        if rc:
            raise ValueError("oracle_rmsnorm_rows rejected its arguments")
        return y, s

    def reference_rmsnorm(self, x, residual, weight, dtype, eps: float, rows=None, threads: int = 0):
        """(y_f64, y_rounded, s_rounded): the FP64 result, its one RNE cast, and the
        rounded residual sums in the storage encoding."""
        y, s = self.rmsnorm_f64(x, residual, weight, dtype, eps, rows=rows, threads=threads)
        return y, self.encode(y, dtype), self.encode(s, dtype)


    def attention_f64(self, q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype, scale: float,
                      causal: bool, rows=None, threads: int = 0):
        """(o_f64, lse_f64): attention of stored [BH, S, d] tensors (views with unit
        column stride allowed); ``rows`` selects flat rows h * Sq + i."""
        a, b, c = (_as_storage(t, dtype) for t in (q, k, v))
        if a.ndim != 3 or b.ndim != 3 or c.ndim != 3:
            raise ValueError("expected [BH, S, d] tensors")
        BH, Sq, d = a.shape
        Sk = b.shape[1]
        if b.shape != (BH, Sk, d) or c.shape != (BH, Sk, d):
            raise ValueError("k and v must be [BH, Sk, d] with q's BH and d")
        es = a.dtype.itemsize
        st = []
        for t in (a, b, c):
            if t.shape[2] > 1 and t.strides[2] != es:
                raise ValueError("the last dimension must be contiguous")
            if any(x % es or x < 0 for x in t.strides[:2]):
                raise ValueError("strides must be non-negative multiples of the element size")
            st += [t.strides[1] // es, t.strides[0] // es]
        nrows = BH * Sq if rows is None else len(rows)
        idx = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        if idx is not None and idx.size and (idx.min() < 0 or idx.max() >= BH * Sq):
            raise IndexError("row index out of range")
        o = np.empty((nrows, d), np.float64)
        lse = np.empty(nrows, np.float64)
        if nrows == 0:
            return o, lse
        rc = self.lib.oracle_attention_rows(
            a.ctypes.data, b.ctypes.data, c.ctypes.data, _code(dtype), BH, Sq, Sk, d, *st,
            float(scale), int(bool(causal)), None if idx is None else idx.ctypes.data, nrows,
            o.ctypes.data_as(_DP), lse.ctypes.data_as(_DP), int(threads))
        if rc:
            raise ValueError("oracle_attention_rows rejected its arguments")
        return o, lse

    def reference_attention(self, q, k, v, dtype, scale, causal, rows=None, threads: int = 0):
        """(o_f64, o_rounded, lse_f64)."""
        o, lse = self.attention_f64(q, k, v, dtype, scale, causal, rows=rows, threads=threads)
        return o, self.encode(o, dtype), lse


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def _load():
    return default().lib


def max_threads() -> int:
    return default().max_threads()


def decode(bits, dtype):
    return default().decode(bits, dtype)


def encode(y, dtype):
    return default().encode(y, dtype)


def softmax_f64(x, dtype, rows=None, threads: int = 0):
    return default().softmax_f64(x, dtype, rows=rows, threads=threads)


def reference(x, dtype, rows=None, threads: int = 0):
    return default().reference(x, dtype, rows=rows, threads=threads)


def softmax_bwd_f64(y, dy, dtype, rows=None, threads: int = 0):
    return default().softmax_bwd_f64(y, dy, dtype, rows=rows, threads=threads)


def reference_bwd(y, dy, dtype, rows=None, threads: int = 0):
    return default().reference_bwd(y, dy, dtype, rows=rows, threads=threads)


def rmsnorm_f64(x, residual, weight, dtype, eps, rows=None, threads: int = 0):
    return default().rmsnorm_f64(x, residual, weight, dtype, eps, rows=rows, threads=threads)


def reference_rmsnorm(x, residual, weight, dtype, eps, rows=None, threads: int = 0):
    return default().reference_rmsnorm(x, residual, weight, dtype, eps, rows=rows, threads=threads)


def attention_f64(q, k, v, dtype, scale, causal, rows=None, threads: int = 0):
    return default().attention_f64(q, k, v, dtype, scale, causal, rows=rows, threads=threads)


def reference_attention(q, k, v, dtype, scale, causal, rows=None, threads: int = 0):
    return default().reference_attention(q, k, v, dtype, scale, causal, rows=rows, threads=threads)
