"""The seeded workload generators: shapes, dtypes, determinism and the value
patterns each recipe promises (no softmax arithmetic is involved)."""
import numpy as np
import torch

import workloads


def test_small_workloads_shapes_and_determinism():
    a = workloads.normal_f32_128x781()
    assert a.shape == (128, 781) and a.dtype == torch.float32
    assert workloads.sha256(a) == workloads.sha256(workloads.normal_f32_128x781())
    b = workloads.normal_bf16_4096x4096(M=64)
    assert b.dtype == torch.bfloat16 and b.shape == (64, 4096)
    assert abs(float(b.float().std()) - 2.0) < 0.05


def test_spiky_rows_have_one_percent_spikes():
    x = workloads.spiky_f16(1000, M=512)
    assert x.dtype == torch.float16
    xf = x.float()
    spikes = xf.abs() == 1e4
    frac = spikes.float().mean().item()
    assert 0.008 < frac < 0.012
    assert torch.all(xf[~spikes].abs() <= 8)
    pos = (xf == 1e4).sum().item()
    neg = (xf == -1e4).sum().item()
    assert abs(pos - neg) < 0.2 * (pos + neg)


def test_offset_rows():
    x = workloads.offset_bf16_64x131072(M=8, N=4096).float()
    means = x.mean(dim=1)
    assert torch.all(means.abs() <= 51)
    assert float((x - means[:, None]).std()) < 1.1


def test_causal_head_mask_and_scale():
    shape = (1, 2, 128, 128, 128)
    h = workloads.causal_head(0, 1, shape=shape).float()
    upper = torch.ones(128, 128, dtype=torch.bool).triu(1)
    assert torch.all(torch.isneginf(h[upper]))
    assert torch.all(torch.isfinite(h[~upper]))
    assert 0.8 < float(h[~upper].std()) < 1.2  # q.k/sqrt(d) has unit variance
    flat = workloads.causal_bf16(shape=shape)
    assert flat.shape == (256, 128)
    assert torch.equal(flat[128:], workloads.causal_head(0, 1, shape=shape))
    picked = workloads.causal_bf16(shape=shape, heads=[1])
    assert torch.equal(picked, flat[128:])


def test_storage_numpy_views():
    t = torch.arange(12, dtype=torch.float32).reshape(3, 4).to(torch.bfloat16)
    s = workloads.storage_numpy(t)
    assert s.dtype == np.uint16 and s.shape == (3, 4)
    assert s[0, 1] == 0x3F80  # 1.0 in bfloat16
    v = workloads.storage_numpy(t[:, 1:3])
    assert v.strides == (8, 2)
