"""Pins for the oracle's fused residual RMSNorm (Warpline README, the description of
its K1 kernel: FP32 residual add rounded once to the input dtype, FP32 RMS reduction,
weight, one rounding of the output), against things other than the oracle's formula:

* the rounded residual sum: bit for bit against torch's own FP32 add and RNE cast;
* torch's float64 ``F.rms_norm`` on that sum with the decoded weight;
* 50-digit ``decimal`` brute force on tiny rows;
* closed forms: constant rows give sign(c) * w, one-hot rows sqrt(N) * sign(a) * w_0;
* invariances: scaling x and r by a power of two leaves y bitwise unchanged (eps = 0),
  a zero residual equals no residual, rows are independent, strided views.
"""
import decimal
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def stored(t):
    return workloads.storage_numpy(t)


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TDT[dt])


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_residual_sum_matches_torch_bitwise(dt):
    # magnitudes spread over many binades, so the FP32 add rounds and the cast rounds
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(64, 257, generator=g) * torch.exp2(torch.randint(-12, 12, (64, 257), generator=g))).to(TDT[dt])
    r = (torch.randn(64, 257, generator=g) * torch.exp2(torch.randint(-30, 4, (64, 257), generator=g))).to(TDT[dt])
    w = rand((257,), dt, 2)
    _, s = oracle.rmsnorm_f64(stored(x), stored(r), stored(w), dt, 1e-6)
    want = (x.float() + r.float()).to(TDT[dt])
    assert np.array_equal(oracle.encode(s, dt), stored(want))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_matches_torch_rms_norm_float64(dt, eps):
    for N in (1, 7, 128, 1000, 4097):
        x, r, w = rand((5, N), dt, N), rand((5, N), dt, N + 1, 0.5), rand((N,), dt, N + 2)
        y, _ = oracle.rmsnorm_f64(stored(x), stored(r), stored(w), dt, eps)
        s = (x.float() + r.float()).to(TDT[dt]).double()
        want = F.rms_norm(s, (N,), weight=w.double(), eps=eps).numpy()
        assert np.allclose(y, want, rtol=1e-13, atol=1e-300), (dt, eps, N)


def _decimal_rmsnorm(s, w, eps):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        sd = [decimal.Decimal(float(v)) for v in s]
        q = sum(v * v for v in sd) / len(sd) + decimal.Decimal(eps)
        den = q.sqrt()
        return np.array([float(v * decimal.Decimal(float(wv)) / den) for v, wv in zip(sd, w)])


def test_decimal_brute_force():
    rng = np.random.default_rng(3)
    for dt in ("f32", "f16", "bf16"):
        for k in range(60):
            N = int(rng.integers(1, 9))
            x, r, w = rand((1, N), dt, 100 + k, 3.0), rand((1, N), dt, 200 + k), rand((N,), dt, 300 + k)
            y, s = oracle.rmsnorm_f64(stored(x), stored(r), stored(w), dt, 1e-5)
            want = _decimal_rmsnorm(s[0], w.double().numpy(), 1e-5)
            assert np.all(np.abs(y[0] - want) <= 1e-14 * np.abs(want) + 1e-300), (dt, k)


def test_closed_forms():
    for dt in ("f32", "bf16"):
        w = rand((64,), dt, 5)
        wd = w.double().numpy()
        for c in (-3.0, 0.5, 2.0):
            x = torch.full((1, 64), c).to(TDT[dt])
            y, _ = oracle.rmsnorm_f64(stored(x), None, stored(w), dt, 0.0)
            assert np.array_equal(y[0], math.copysign(1.0, c) * wd)
        x = torch.zeros(1, 64).to(TDT[dt])
        x[0, 0] = -1.5
        y, _ = oracle.rmsnorm_f64(stored(x), None, stored(w), dt, 0.0)
        assert y[0, 0] == -8.0 * wd[0] and np.all(y[0, 1:] == 0)  # sqrt(64) = 8


def test_scale_invariance_and_zero_residual():
    x, r, w = rand((8, 300), "f32", 1), rand((8, 300), "f32", 2), rand((300,), "f32", 3)
    y1, _ = oracle.rmsnorm_f64(stored(x), stored(r), stored(w), "f32", 0.0)
    y2, _ = oracle.rmsnorm_f64(stored(x * 8), stored(r * 8), stored(w), "f32", 0.0)
    assert np.array_equal(y1, y2)
    a, _ = oracle.rmsnorm_f64(stored(x), None, stored(w), "f32", 1e-6)
    b, _ = oracle.rmsnorm_f64(stored(x), stored(torch.zeros_like(x)), stored(w), "f32", 1e-6)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_strided_views_and_rows(dt):
    xb, rb, w = rand((9, 70), dt, 1), rand((9, 90), dt, 2), rand((50,), dt, 3)
    xv, rv = stored(xb)[:, 3:53], stored(rb)[:, 10:60]
    y, s = oracle.rmsnorm_f64(xv, rv, stored(w), dt, 1e-6)
    y2, s2 = oracle.rmsnorm_f64(np.ascontiguousarray(xv), np.ascontiguousarray(rv), stored(w), dt, 1e-6)
    assert np.array_equal(y, y2) and np.array_equal(s, s2)
    y3, _ = oracle.rmsnorm_f64(xv, rv, stored(w), dt, 1e-6, rows=[7, 0, 3])
    assert np.array_equal(y3, y[[7, 0, 3]])


def test_special_values():
    x = torch.tensor([[1.0, float("nan"), 2.0], [0.0, 0.0, 0.0], [float("inf"), 1.0, 1.0]])
    w = torch.ones(3)
    y, _ = oracle.rmsnorm_f64(stored(x), None, stored(w), "f32", 0.0)
    assert np.all(np.isnan(y[0])) and np.all(np.isnan(y[1]))  # NaN poisons q; 0/0
    y, _ = oracle.rmsnorm_f64(stored(x), None, stored(w), "f32", 1e-6)
    assert np.all(y[1] == 0.0)                                   # eps > 0: a zero row stays 0
    assert np.isnan(y[2, 0]) and np.all(y[2, 1:] == 0.0)         # inf / inf, finite / inf
