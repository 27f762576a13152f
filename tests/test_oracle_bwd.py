"""Pins for the oracle's softmax backward, dx = y * (dy - sum(y * dy)) ("Measured
optimization case studies", section "Training: backward kernels through autograd"),
against things other than the oracle's own formula:

* central finite differences of L(x) = sum_j dy_j softmax(x)_j, with the softmax taken
  from the oracle's forward pass (an independent code path);
* torch's float64 softmax backward on the same decoded y and dy;
* algebra: sum_j dx_j = d (1 - sum_j y_j), linearity in dy, one-hot y gives 0,
  a constant dy gives c y (1 - sum y);
* strided views, row subsets and independence of rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def stored(x, dtype):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(TORCH_DT[dtype])
    return workloads.storage_numpy(t)


def test_matches_finite_differences_of_the_forward_oracle():
    rng = np.random.default_rng(20)
    h = 2.0 ** -12
    for n in (2, 5, 17, 64):
        # logits on a 1/8 grid so that x +/- h is exact in FP32
        x = (rng.integers(-32, 33, size=(1, n)) / 8.0).astype(np.float32)
        g = rng.standard_normal((1, n)).astype(np.float32)
        y = oracle.softmax_f64(x, "f32")
        dx = oracle.softmax_bwd_f64(y.astype(np.float32), g, "f32")[0]
        fd = np.empty(n)
        for i in range(n):
            xp, xm = x.copy(), x.copy()
            xp[0, i] += np.float32(h)
            xm[0, i] -= np.float32(h)
            lp = float(oracle.softmax_f64(xp, "f32")[0] @ g[0].astype(np.float64))
            lm = float(oracle.softmax_f64(xm, "f32")[0] @ g[0].astype(np.float64))
            fd[i] = (lp - lm) / (2 * h)
        scale = np.abs(y[0] * g[0]).sum()
        assert np.max(np.abs(dx - fd)) <= 1e-6 * scale, (n, dx, fd)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_matches_torch_float64_softmax_backward(dtype):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((32, 700)) * 3
    ys = stored(torch.softmax(torch.from_numpy(x), -1).numpy(), dtype)
    gs = stored(rng.standard_normal((32, 700)), dtype)
    dx = oracle.softmax_bwd_f64(ys, gs, dtype)
    yt = torch.from_numpy(oracle.decode(ys, dtype))
    gt = torch.from_numpy(oracle.decode(gs, dtype))
    want = torch._softmax_backward_data(gt, yt, -1, torch.float64).numpy()
    scale = (yt.abs() * (gt.abs() + (yt * gt).sum(-1, keepdim=True).abs())).numpy()
    assert np.all(np.abs(dx - want) <= 1e-14 * scale + 1e-300)


def test_algebraic_identities():
    rng = np.random.default_rng(22)
    y = stored(torch.softmax(torch.randn(16, 300, dtype=torch.float64) * 2, -1).numpy(), "f32")
    g1 = rng.standard_normal((16, 300)).astype(np.float32)
    g2 = rng.standard_normal((16, 300)).astype(np.float32)
    yd = y.astype(np.float64)
    d1 = oracle.softmax_bwd_f64(y, g1, "f32")
    # sum_j dx_j = d (1 - sum_j y_j)
    d = (yd * g1).sum(1)
    assert np.allclose(d1.sum(1), d * (1 - yd.sum(1)), rtol=0, atol=1e-13)
    # linear in dy (2 g1 - g2 is exact in FP32 for these magnitudes up to one rounding)
    g3 = (2 * g1.astype(np.float64) - g2).astype(np.float32)
    d3 = oracle.softmax_bwd_f64(y, g3, "f32")
    d2 = oracle.softmax_bwd_f64(y, g2, "f32")
    lin = oracle.softmax_bwd_f64(y, (g3.astype(np.float64)).astype(np.float32), "f32")
    assert np.array_equal(d3, lin)
    assert np.allclose(d3, 2 * d1 - d2, rtol=0, atol=1e-6 * np.abs(yd).max())
    # a constant upstream gradient c gives c y (1 - sum y), which is ~0
    c = np.full((16, 300), 1.75, np.float32)
    dc = oracle.softmax_bwd_f64(y, c, "f32")
    assert np.allclose(dc, 1.75 * yd * (1 - yd.sum(1, keepdims=True)), rtol=1e-12, atol=1e-300)
    # one-hot y gives exactly 0
    oh = np.zeros((3, 50), np.float32)
    oh[[0, 1, 2], [0, 20, 49]] = 1
    assert np.all(oracle.softmax_bwd_f64(oh, rng.standard_normal((3, 50)).astype(np.float32), "f32") == 0)


def test_two_element_closed_form():
    # y = [p, 1-p]: dx_0 = p (1-p) (g0 - g1) = -dx_1
    p = np.float32(0.375)
    y = np.array([[p, 1 - p]], np.float32)
    g = np.array([[2.5, -1.0]], np.float32)
    dx = oracle.softmax_bwd_f64(y, g, "f32")[0]
    assert dx[0] == pytest.approx(0.375 * 0.625 * 3.5, rel=1e-15)
    assert dx[1] == pytest.approx(-dx[0], rel=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_views_and_rows(dtype):
    rng = np.random.default_rng(23)
    yb = stored(rng.random((20, 333)), dtype)
    gb = stored(rng.standard_normal((20, 350)), dtype)
    yv, gv = yb[:, :300], gb[:, 10:310]
    full = oracle.softmax_bwd_f64(yv, gv, dtype)
    assert np.array_equal(full, oracle.softmax_bwd_f64(np.ascontiguousarray(yv),
                                                       np.ascontiguousarray(gv), dtype))
    assert np.array_equal(oracle.softmax_bwd_f64(yv, gv, dtype, rows=[19, 3, 3]), full[[19, 3, 3]])
    assert np.array_equal(full[7], oracle.softmax_bwd_f64(yv[7:8], gv[7:8], dtype)[0])


def test_nan_propagates():
    y = np.array([[0.5, 0.5], [0.25, 0.75]], np.float32)
    g = np.array([[np.nan, 1.0], [1.0, 2.0]], np.float32)
    dx = oracle.softmax_bwd_f64(y, g, "f32")
    assert np.all(np.isnan(dx[0])) and np.all(np.isfinite(dx[1]))
