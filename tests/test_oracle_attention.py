"""Pins for the oracle's attention, O = softmax(scale * Q K^T [causal]) V per (head,
query) row in FP64, against things other than its own formula:

* torch's float64 ``scaled_dot_product_attention`` (an explicit bottom-right causal mask
  when Sq != Sk), and its log-sum-exp against ``torch.logsumexp``;
* 50-digit ``decimal`` brute force on tiny heads;
* closed forms: identical keys give the mean of the visible value rows; the first query
  of a square causal head returns v_0 exactly; two visible keys give logistic weights;
* a fully masked query (Sq > Sk, causal) gives zeros and lse = -inf;
* strided views (a head stride larger than S * d, a row stride larger than d), row subsets.
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


def st(t):
    return workloads.storage_numpy(t.contiguous())


def rand(shape, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(TDT[dt])


def causal_mask(Sq, Sk):
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Sk)[None, :]
    return j <= i + (Sk - Sq)  # True = visible


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk,d", [(16, 16, 8), (33, 47, 64), (64, 64, 128), (40, 24, 32)])
def test_matches_torch_sdpa_float64(dt, causal, Sq, Sk, d):
    BH = 3
    q, k, v = rand((BH, Sq, d), dt, 1), rand((BH, Sk, d), dt, 2), rand((BH, Sk, d), dt, 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention_f64(st(q), st(k), st(v), dt, scale, causal)
    mask = causal_mask(Sq, Sk) if causal else torch.ones(Sq, Sk, dtype=torch.bool)
    vis = mask.any(dim=1)  # torch gives NaN for a fully masked query; compared separately
    want = F.scaled_dot_product_attention(q.double(), k.double(), v.double(), attn_mask=mask,
                                          scale=scale)
    o = o.reshape(BH, Sq, d)
    assert np.allclose(o[:, vis.numpy()], want[:, vis].numpy(), rtol=1e-12, atol=1e-14)
    assert np.all(o[:, ~vis.numpy()] == 0.0)
    s = torch.einsum("hid,hjd->hij", q.double(), k.double()) * scale
    s = s.masked_fill(~mask, -math.inf)
    wl = torch.logsumexp(s, dim=-1).numpy()
    lse = lse.reshape(BH, Sq)
    assert np.allclose(lse[:, vis.numpy()], wl[:, vis.numpy()], rtol=1e-13, atol=1e-13)
    assert np.all(np.isneginf(lse[:, ~vis.numpy()]))


def _decimal_attention(q, k, v, scale, causal):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        Sq, d = q.shape
        Sk = k.shape[0]
        out = np.zeros((Sq, d))
        for i in range(Sq):
            s = []
            for j in range(Sk):
                if causal and j > i + (Sk - Sq):
                    s.append(None)
                    continue
                s.append(decimal.Decimal(scale) * sum(decimal.Decimal(float(q[i, c])) *
                                                      decimal.Decimal(float(k[j, c])) for c in range(d)))
            fin = [x for x in s if x is not None]
            if not fin:
                continue
            m = max(fin)
            e = [decimal.Decimal(0) if x is None else (x - m).exp() for x in s]
            tot = sum(e)
            for c in range(d):
                out[i, c] = float(sum(e[j] * decimal.Decimal(float(v[j, c])) for j in range(Sk)) / tot)
        return out


def test_decimal_brute_force():
    for seed in range(12):
        causal = bool(seed % 2)
        q, k, v = rand((1, 4, 3), "bf16", seed, 2), rand((1, 5, 3), "bf16", seed + 50, 2), rand((1, 5, 3), "bf16", seed + 99)
        o, _ = oracle.attention_f64(st(q), st(k), st(v), "bf16", 0.7, causal)
        want = _decimal_attention(q[0].double().numpy(), k[0].double().numpy(), v[0].double().numpy(), 0.7, causal)
        assert np.allclose(o, want, rtol=1e-14, atol=1e-15), seed


def test_closed_forms():
    d = 16
    k = rand((1, 1, d), "f32", 1).expand(1, 9, d).contiguous()  # identical keys
    q, v = rand((1, 9, d), "f32", 2), rand((1, 9, d), "f32", 3)
    o, lse = oracle.attention_f64(st(q), st(k), st(v), "f32", 0.25, True)
    vd = v[0].double().numpy()
    for i in range(9):
        assert np.allclose(o[i], vd[: i + 1].mean(axis=0), rtol=1e-14, atol=1e-15)
    assert np.array_equal(o[0], vd[0])  # the first query sees only key 0: exactly v_0
    # two keys: logistic weights
    q, k, v = rand((1, 1, d), "f32", 4), rand((1, 2, d), "f32", 5), rand((1, 2, d), "f32", 6)
    o, _ = oracle.attention_f64(st(q), st(k), st(v), "f32", 0.5, False)
    s = 0.5 * (k[0].double() @ q[0, 0].double()).numpy()
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    assert np.allclose(o[0], p0 * v[0, 0].double().numpy() + (1 - p0) * v[0, 1].double().numpy(),
                       rtol=1e-14, atol=1e-15)


def test_strided_views_and_rows():
    qb, kb, vb = rand((2, 10, 40), "bf16", 1), rand((2, 12, 48), "bf16", 2), rand((3, 12, 32), "bf16", 3)
    qv, kv, vv = st(qb)[:, 2:8, 4:36], st(kb)[:, :, 8:40], st(vb)[1:3]
    o, lse = oracle.attention_f64(qv, kv, vv, "bf16", 0.2, True)
    o2, lse2 = oracle.attention_f64(np.ascontiguousarray(qv), np.ascontiguousarray(kv),
                                    np.ascontiguousarray(vv), "bf16", 0.2, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    o3, _ = oracle.attention_f64(qv, kv, vv, "bf16", 0.2, True, rows=[11, 0, 5])
    assert np.array_equal(o3, o[[11, 0, 5]])
