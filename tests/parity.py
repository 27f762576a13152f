"""Comparison of GPU outputs with the FP64 oracle (helper for the GPU tests).

Rule (Warpline README, its correctness-check paragraph): an output g passes
when |g - r| <= atol + rtol * |r|, with r the oracle's FP64 result rounded once
to the storage dtype. Tolerances:

* FP16 and BF16: atol = rtol = 4e-3 (the BF16 softmax tolerance that README
  lists, applied to FP16 as well);
* FP32: rtol = 1e-6 against the FP64 result itself (not its rounding), with
  atol = 2^-126 (the smallest normal FP32) so that results that underflow
  compare absolutely.

Positions where the oracle gives NaN must be NaN on the GPU and vice versa.
The helper also reports the maximum absolute error against the FP64 result and
a relative error taken only where |y| > 1e-3 (the README's thresholded
relative error).

A second, tighter gate applies to FP16 and BF16 (the README's tolerance is the
stated bar; this one catches what its absolute term hides on probabilities of
1e-4 to 1e-3): |g - r| <= ulp(r) + f, one unit in the last place of the dtype at
r. The kernels form y in FP32 (a few FP32 ulps from the exact value) and round
once, so they land on r or on its neighbour. f is 0 for FP16 and 2^-126 for BF16:
BF16 shares FP32's exponent range, and the FP32 exponential flushes results below
the smallest normal FP32 to zero, where r may still be a BF16 subnormal.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads

TOL = {"f32": (2.0 ** -126, 1e-6), "f16": (4e-3, 4e-3), "bf16": (4e-3, 4e-3)}
# (fraction bits, smallest normal exponent, floor f) of the one-ulp gate
ULP_GATE = {"f16": (10, -14, 0.0), "bf16": (7, -126, 2.0 ** -126)}


def _ulp_t(r: torch.Tensor, dt: str) -> torch.Tensor:
    p, emin, _ = ULP_GATE[dt]
    a = r.abs()
    _, ex = torch.frexp(a)               # |r| = f * 2^ex, f in [0.5, 1); e = ex - 1
    e = torch.where(a == 0, torch.full_like(ex, emin), torch.clamp(ex - 1, min=emin))
    # 2^(e - p) built from its FP64 exponent field (exact; e - p >= -133)
    return ((e.to(torch.int64) - p + 1023) << 52).view(torch.float64)


def ulp(r, dt: str):
    """Spacing of the FP16/BF16 grid at |r| (r on that grid): 2^(e - p) for
    2^e <= |r| < 2^(e+1), the subnormal spacing below the normal range and at 0.
    Takes and returns numpy arrays or torch tensors (float64)."""
    if isinstance(r, np.ndarray):
        return _ulp_t(torch.from_numpy(np.ascontiguousarray(r, dtype=np.float64)), dt).numpy()
    return _ulp_t(r.double(), dt)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def _worst(score: torch.Tensor):
    flat = int(torch.argmax(score))
    return divmod(flat, score.shape[1]) if score.dim() == 2 else (flat, 0)


def compare(g: torch.Tensor, x: torch.Tensor, rows=None, what: str = "") -> dict:
    """Check GPU result ``g`` (rows x N, any device) against the oracle for the CPU
    input ``x`` (M x N; ``rows`` selects the rows ``g`` holds). Raises AssertionError.
    The element-wise arithmetic runs in torch's multi-threaded CPU kernels (the
    workloads reach 10^9 elements)."""
    dt = workloads.dtype_name(x)
    y_np, yr = oracle.reference(workloads.storage_numpy(x), dt, rows=rows)
    y = torch.from_numpy(y_np)
    ref = y if dt == "f32" else torch.from_numpy(oracle.decode(yr, dt))
    gd = g.detach().cpu().double().reshape(ref.shape)
    atol, rtol = TOL[dt]
    nan_ref, nan_g = ref.isnan(), gd.isnan()
    assert torch.equal(nan_ref, nan_g), \
        f"{what}: NaN pattern differs ({int(nan_ref.sum())} vs {int(nan_g.sum())})"
    n = ref.numel() - int(nan_ref.sum())
    err = (gd - ref).abs_().masked_fill_(nan_ref, 0.0)
    bound = ref.abs().mul_(rtol).add_(atol).masked_fill_(nan_ref, 1.0)
    frac = err / bound
    bad = frac > 1.0
    if bool(bad.any()):
        i, j = _worst(frac)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {n} outside tolerance; worst at ({i},{j}): "
            f"gpu={float(gd[i, j])!r} ref={float(ref[i, j])!r} y={float(y[i, j])!r}")
    max_ulp = None
    if dt != "f32":
        u = _ulp_t(ref, dt).masked_fill_(nan_ref, 1.0)
        in_ulps = err / u
        ubad = err > u + ULP_GATE[dt][2]
        if bool(ubad.any()):
            i, j = _worst(torch.where(ubad, in_ulps, torch.full_like(in_ulps, -1.0)))
            raise AssertionError(
                f"{what}: {int(ubad.sum())} of {n} more than one ulp from the rounded "
                f"oracle; worst at ({i},{j}): gpu={float(gd[i, j])!r} ref={float(ref[i, j])!r} "
                f"y={float(y[i, j])!r}")
        max_ulp = float(in_ulps.max()) if n else 0.0
    fin = ~nan_ref & y.isfinite()
    abs_err = (gd - y).abs_().masked_fill_(~fin, 0.0)
    big = fin & (y.abs() > 1e-3)
    rel = (abs_err / y.abs()).masked_fill_(~big, 0.0)
    return {"max_abs": float(abs_err.max()) if n else 0.0,
            "max_rel_thr": float(rel.max()) if n else 0.0,
            "worst_frac_of_tol": float(frac.max()) if n else 0.0,
            "max_ulp_vs_rounded": max_ulp, "n": n}


def rel_thr_bound(dt: str) -> float:
    """Bound on the thresholded relative error (|y| > 1e-3) against the FP64 result:
    one rounding to the dtype (half an ulp) plus the one-ulp gate's neighbour, at most
    1.5 ulp, i.e. below 2^(1-p) relative with p fraction bits (FP16 10, BF16 7);
    FP32: the 1e-6 relative tolerance."""
    return {"f16": 2.0 ** -9, "bf16": 2.0 ** -6, "f32": 1e-6}[dt]


def row_sum_bound(dt: str) -> float:
    """|sum_j g_j - 1| bound per row: half a unit in the last place of the output
    dtype for every rounding, plus 1e-5 slack (FP32: 2e-5, the row-normalisation
    tolerance of "Measured optimization case studies", section "CUDA: parallel
    reduction, online statistics and a numerical fix")."""
    return {"bf16": 2.0 ** -8 + 1e-5, "f16": 2.0 ** -11 + 1e-5, "f32": 2e-5}[dt]


# ------------------------------------------------------------------ backward
# dx = y * (dy - d), d = sum_k y_k dy_k. Both sides read the same stored y and dy;
# the GPU forms d in FP32 and rounds dx once, the oracle works in FP64. The pages
# give no backward tolerance, so it is derived from that arithmetic. Error scale
# per element: s_j = |y_j| (|dy_j| + sum_k |y_k dy_k|) >= |dx_j|. An FP32 dot over
# a lane's V*E elements and a log2(G)-deep tree is off by at most about
# (V*E + log2 G) * 2^-24 * sum|y dy| (< 3e-6 s_j for every one-pass shape; the
# compensated FP32 dot far less), so 1e-4 s_j bounds the FP32 error with margin
# while a wrong sign, index or term (an error of order s_j) still fails.
#   FP16/BF16: |g - r| <= u |r| + 1e-4 s_j + a
#       r: the oracle rounded once to the dtype; u = 2^-10 (FP16) / 2^-7 (BF16), one
#       unit in the last place relative to |r|: the FP32 value may sit on the other
#       side of a rounding boundary; a: the dtype's subnormal spacing.
#   FP32:      |g - dx| <= 1e-6 (|dx| + s_j) + 2^-126   (dx: the FP64 result)
TOL_BWD = {"f32": (1e-6, 1e-6, 2.0 ** -126), "f16": (2.0 ** -10, 1e-4, 2.0 ** -24),
           "bf16": (2.0 ** -7, 1e-4, 2.0 ** -133)}


def compare_bwd(g: torch.Tensor, y: torch.Tensor, dy: torch.Tensor, rows=None,
                what: str = "") -> dict:
    dt = workloads.dtype_name(y)
    ys, ds = workloads.storage_numpy(y), workloads.storage_numpy(dy)
    dx, dxr = oracle.reference_bwd(ys, ds, dt, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    yd = torch.from_numpy(oracle.decode(np.ascontiguousarray(ys)[sel], dt))
    dd = torch.from_numpy(oracle.decode(np.ascontiguousarray(ds)[sel], dt))
    # error scale s_j = |y_j| (|dy_j| + sum_k |y_k dy_k|)
    s = yd.abs() * (dd.abs() + (yd * dd).abs_().sum(dim=1, keepdim=True))
    ref = torch.from_numpy(dx if dt == "f32" else oracle.decode(dxr, dt))
    gd = g.detach().cpu().double().reshape(ref.shape)
    rt, sc, at = TOL_BWD[dt]
    nan_ref, nan_g = ref.isnan(), gd.isnan()
    assert torch.equal(nan_ref, nan_g), \
        f"{what}: NaN pattern differs ({int(nan_ref.sum())} vs {int(nan_g.sum())})"
    inf_ref = ref.isinf()
    assert torch.equal(gd[inf_ref], ref[inf_ref]), f"{what}: infinities differ"
    skip = nan_ref | inf_ref
    n = ref.numel() - int(skip.sum())
    err = (gd - ref).abs_().masked_fill_(skip, 0.0)
    bound = (ref.abs().mul_(rt) + s.mul_(sc)).add_(at).masked_fill_(skip, 1.0)
    frac = err / bound
    bad = frac > 1.0
    if bool(bad.any()):
        i, j = _worst(frac)
        raise AssertionError(f"{what}: {int(bad.sum())} of {n} outside tolerance; worst at "
                             f"({i},{j}): gpu={float(gd[i, j])!r} ref={float(ref[i, j])!r} "
                             f"bound={float(bound[i, j])!r}")
    return {"max_abs": float(err.max()) if n else 0.0,
            "worst_frac_of_tol": float(frac.max()) if n else 0.0, "n": n}


# ------------------------------------------------------------------ residual RMSNorm
# The GPU forms s = x + r in FP32 and rounds once (equal to the correctly rounded
# sum for every dtype here, so s must match the oracle bit for bit), sums s^2 in FP32
# (compensated for FP32 data), and rounds y once. The FP32 value of y is within about
# 1e-6 relative of the FP64 one, so the rounded result is the oracle's rounding or
# its neighbour:
#   FP16/BF16: |g - r| <= u |r| + a   (u = 2^-10 / 2^-7, one unit in the last place
#              relative to |r|; a the dtype's subnormal spacing)
#   FP32:      |g - y| <= 1e-6 |y| + 2^-126   (y the FP64 result)
# (The pages' own BF16 tolerance for this kernel, 0.02 absolute and relative, is
# looser than both.)
TOL_RMS = {"f32": (1e-6, 2.0 ** -126), "f16": (2.0 ** -10, 2.0 ** -24), "bf16": (2.0 ** -7, 2.0 ** -133)}


def compare_rms(g: torch.Tensor, x: torch.Tensor, r, w: torch.Tensor, eps: float, s_gpu=None,
                rows=None, what: str = "") -> dict:
    dt = workloads.dtype_name(x)
    rs = None if r is None else workloads.storage_numpy(r)
    y, yr, sr = oracle.reference_rmsnorm(workloads.storage_numpy(x), rs, workloads.storage_numpy(w),
                                         dt, eps, rows=rows)
    if s_gpu is not None:
        sg = workloads.storage_numpy(s_gpu.detach().cpu().contiguous())
        assert np.array_equal(sg, sr), f"{what}: residual_out differs from the rounded sum"
    gd = to_f64(g)
    ref = y if dt == "f32" else oracle.decode(yr, dt)
    rt, at = TOL_RMS[dt]
    nan_ref, nan_g = np.isnan(ref), np.isnan(gd)
    assert np.array_equal(nan_ref, nan_g), f"{what}: NaN pattern differs ({nan_ref.sum()} vs {nan_g.sum()})"
    inf_ref = np.isinf(ref)
    assert np.array_equal(gd[inf_ref], ref[inf_ref]), f"{what}: infinities differ"
    ok = ~nan_ref & ~inf_ref
    err = np.abs(gd[ok] - ref[ok])
    bound = rt * np.abs(ref[ok]) + at
    bad = err > bound
    if bad.any():
        idx = np.argwhere(ok)[np.argmax(err - bound)]
        i, j = int(idx[0]), int(idx[1])
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at "
                             f"({i},{j}): gpu={gd[i, j]!r} ref={ref[i, j]!r}")
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "worst_frac_of_tol": float(np.max(err / bound)) if err.size else 0.0, "n": int(err.size)}


# ------------------------------------------------------------------ fused attention
# The kernel forms the scores in FP32 (exact products of 16-bit inputs), the row
# statistics in FP32, and rounds the probabilities to the input dtype before the
# product with V (the FlashAttention contract). Rounding P moves o_i by at most
# 2^-(p+1) * sum_j P_ij |v_j| (p fraction bits), so with a factor 4 of margin:
#   |g - r| <= u |r| + c * sum_j P_ij |v_jd| + a,
# u one unit in the last place relative (2^-7 BF16, 2^-10 FP16), c = 2^-7 (BF16) /
# 2^-10 (FP16), a the subnormal spacing; sum_j P |v| is the oracle's attention of |v|.
# A wrong mask, scale or index moves o by the order of sum_j P |v| and fails.
TOL_ATTN = {"f16": (2.0 ** -10, 2.0 ** -10, 2.0 ** -24), "bf16": (2.0 ** -7, 2.0 ** -7, 2.0 ** -133)}


def compare_attn(g: torch.Tensor, q, k, v, scale: float, causal: bool, rows=None, lse_gpu=None,
                 what: str = "") -> dict:
    dt = workloads.dtype_name(q)
    qs, ks, vs = (workloads.storage_numpy(t.detach().cpu().contiguous()) for t in (q, k, v))
    o, orr, lse = oracle.reference_attention(qs, ks, vs, dt, scale, causal, rows=rows)
    vabs = vs & np.uint16(0x7FFF)
    mag, _ = oracle.attention_f64(qs, ks, vabs, dt, scale, causal, rows=rows)
    gd = to_f64(g).reshape(o.shape)
    ref = oracle.decode(orr, dt)
    u, c, a = TOL_ATTN[dt]
    assert not np.isnan(gd).any(), f"{what}: NaN in the output"
    err = np.abs(gd - ref)
    bound = u * np.abs(ref) + c * mag + a
    bad = err > bound
    if bad.any():
        i, j = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst at "
                             f"({i},{j}): gpu={gd[i, j]!r} ref={ref[i, j]!r} scale={mag[i, j]!r}")
    if lse_gpu is not None:
        lg = lse_gpu.detach().cpu().double().numpy().reshape(-1)
        fin = np.isfinite(lse)
        assert np.array_equal(np.isneginf(lg), ~fin), f"{what}: lse -inf pattern differs"
        assert np.allclose(lg[fin], lse[fin], rtol=2e-6, atol=2e-6), f"{what}: lse differs"
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "worst_frac_of_tol": float(np.max(err / bound)) if err.size else 0.0, "n": int(err.size)}
