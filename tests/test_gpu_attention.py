"""GPU parity of the fused attention forward (sm_attention_fwd) against the FP64 oracle:
head dims 64 and 128, causal and not, Sq = Sk and Sq != Sk (queries that see no key),
ragged lengths, strided head layouts, log-sum-exp, repeatability, torch's FP32 SDPA,
and the attention-shaped workload (8 x 32 heads, 2048 x 2048, d = 128) at full size,
whole heads against the oracle."""
import math

import numpy as np
import pytest
import torch

import memory_bound_row_sm_amd as sm
import workloads
from parity import compare_attn, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    sm.lib()


def qkv(BH, Sq, Sk, d, dt, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(BH, Sq, d, generator=g) * scale).to(TDT[dt])
    k = (torch.randn(BH, Sk, d, generator=g) * scale).to(TDT[dt])
    v = torch.randn(BH, Sk, d, generator=g).to(TDT[dt])
    return q, k, v


def run(q, k, v, causal, scale=None, lse=False):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.full_like(qd, float("nan"))
    ls = torch.full((q.shape[0] * q.shape[1],), float("nan"), device=DEV) if lse else None
    sm.attention(qd, kd, vd, scale=scale, causal=causal, out=o, lse=ls)
    torch.cuda.synchronize()
    return o, ls


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("BH,Sq,Sk", [(2, 128, 128), (3, 200, 333), (1, 1, 1), (2, 257, 64),
                                      (1, 64, 1000), (2, 130, 70)])
def test_shapes(dt, d, causal, BH, Sq, Sk):
    q, k, v = qkv(BH, Sq, Sk, d, dt, seed=Sq * 7 + Sk)
    scale = 1.0 / math.sqrt(d)
    o, ls = run(q, k, v, causal, scale, lse=True)
    st = compare_attn(o, q, k, v, scale, causal, lse_gpu=ls, what=f"{dt} d={d} causal={causal} {BH}x{Sq}x{Sk}")
    assert st["worst_frac_of_tol"] <= 1.0
    if causal and Sq > Sk:  # queries i < Sq - Sk see no key
        n = Sq - Sk
        assert (o[:, :n].float() == 0).all()
        assert torch.isneginf(ls.view(BH, Sq)[:, :n]).all()


def test_large_scores_and_scale():
    """Scores of magnitude ~100 (sharp softmax) and a non-default scale."""
    q, k, v = qkv(2, 300, 300, 128, "bf16", seed=5, scale=3.0)
    for causal in (False, True):
        o, ls = run(q, k, v, causal, scale=0.3, lse=True)
        compare_attn(o, q, k, v, 0.3, causal, lse_gpu=ls, what=f"sharp causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_negative_and_zero_scale(causal):
    """A negative scale (folded into the sign of Q) and scale 0 (uniform weights over the
    visible keys)."""
    q, k, v = qkv(3, 200, 260, 64, "bf16", seed=21)
    for scale in (-0.125, -1.5, 0.0):
        o, ls = run(q, k, v, causal, scale=scale, lse=True)
        compare_attn(o, q, k, v, scale, causal, lse_gpu=ls, what=f"scale={scale} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_item_order_over_many_workgroups(causal):
    """Grids of 15 and 30 work items (not multiples of the 8 XCDs), an odd q-block count
    (the middle q-block of a head has no causal partner) and Sq != Sk."""
    for BH, Sq, Sk in [(5, 700, 700), (3, 1300, 1500), (2, 640, 129)]:
        q, k, v = qkv(BH, Sq, Sk, 128, "f16", seed=BH * Sq)
        o, ls = run(q, k, v, causal, lse=True)
        compare_attn(o, q, k, v, 1.0 / math.sqrt(128), causal, lse_gpu=ls,
                     what=f"{BH}x{Sq}x{Sk} causal={causal}")


def test_strided_heads():
    """q, k, v as [1, S, H, d] tensors viewed as [H, S, d] (row stride H * d, head stride d)."""
    H, S, d = 4, 160, 64
    g = torch.Generator().manual_seed(11)
    base = [torch.randn(1, S, H, d, generator=g).to(torch.bfloat16) for _ in range(3)]
    views = [b.to(DEV).transpose(1, 2)[0] for b in base]  # [H, S, d], strided
    o = torch.full((H, S, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    sm.attention(*views, causal=True, out=o)
    torch.cuda.synchronize()
    cpu = [b.transpose(1, 2)[0].contiguous() for b in base]
    compare_attn(o, *cpu, 1.0 / math.sqrt(d), True, what="strided heads")


def test_repeatable_and_torch_fp32():
    q, k, v = qkv(4, 512, 512, 128, "bf16", seed=3)
    a, _ = run(q, k, v, True)
    b, _ = run(q, k, v, True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    want = torch.nn.functional.scaled_dot_product_attention(q.float(), k.float(), v.float(), is_causal=True)
    assert float((a.float().cpu() - want).abs().max()) < 2e-2


def test_no_keys_and_no_queries():
    """Sk = 0: every query sees no key (zeros, lse = -inf); Sq = 0: nothing to do."""
    q = torch.randn(3, 70, 64).to(torch.bfloat16)
    k = torch.empty(3, 0, 64, dtype=torch.bfloat16)
    for causal in (False, True):
        o, ls = run(q, k, k.clone(), causal, lse=True)
        assert (o.float() == 0).all() and torch.isneginf(ls).all()
    qe = torch.empty(2, 0, 128, device=DEV, dtype=torch.float16)
    ke = torch.randn(2, 5, 128, device=DEV).half()
    oe = torch.empty_like(qe)
    sm.attention(qe, ke, ke, causal=True, out=oe)
    torch.cuda.synchronize()


ATTN_WL = (8 * 32, 2048, 128)   # heads, queries = keys, head dim
ATTN_CHUNK = 64                  # heads per oracle comparison
# every head compared whole against the oracle, in BF16 (the bench's dtype) and FP16
ATTN_CASES = [(dt, h0) for dt in ("bf16", "f16") for h0 in range(0, ATTN_WL[0], ATTN_CHUNK)]
_attn_cache = {}


def attention_workload(dt):
    """8 x 32 heads, 2048 queries and keys, d = 128, causal: q, k, v ~ N(0, 1) from
    seed 2026, rounded to ``dt``; the kernel's output and lse (run once per dtype)."""
    if dt not in _attn_cache:
        _attn_cache.clear()
        BH, S, d = ATTN_WL
        g = torch.Generator().manual_seed(2026)
        q = torch.randn(BH, S, d, generator=g).to(TDT[dt])
        k = torch.randn(BH, S, d, generator=g).to(TDT[dt])
        v = torch.randn(BH, S, d, generator=g).to(TDT[dt])
        o, ls = run(q, k, v, True, lse=True)
        _attn_cache[dt] = (q, k, v, o.cpu(), ls.cpu())
    return _attn_cache[dt]


@pytest.mark.parametrize("dt,h0", ATTN_CASES)
def test_attention_workload_full_size(dt, h0):
    """The attention workload in the bench's launch configuration, every query row of
    heads h0 .. h0 + 63 against the oracle."""
    q, k, v, o, ls = attention_workload(dt)
    BH, S, d = ATTN_WL
    h1 = min(BH, h0 + ATTN_CHUNK)
    st = compare_attn(o[h0:h1], q[h0:h1], k[h0:h1], v[h0:h1], 1.0 / math.sqrt(d), True,
                      lse_gpu=ls.view(BH, S)[h0:h1], what=f"attention workload {dt} heads {h0}:{h1}")
    log(f"[attn] workload {dt} heads {h0}:{h1} ({(h1 - h0) * S} rows): {st}")
    # the first query of every head sees only key 0: o = v_0 rounded
    assert torch.equal(o[h0:h1, 0].view(torch.int16), v[h0:h1, 0].view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
def test_running_maximum_grows_along_the_keys(causal):
    """Keys scaled by 1 + 6 j / Sk, so most queries' running maximum passes the lazy margin
    block after block; then one late key aligned with every query, whose score lies about
    a hundred binades above the others (the accumulated O and l are rescaled by ~2^-100)."""
    BH, S, d = 2, 700, 128
    q, k, v = qkv(BH, S, S, d, "bf16", seed=31)
    ramp = (1 + 6 * torch.arange(S, dtype=torch.float32) / S).view(1, S, 1)
    k2 = (k.float() * ramp).to(torch.bfloat16)
    o, ls = run(q, k2, v, causal, scale=0.3, lse=True)
    compare_attn(o, q, k2, v, 0.3, causal, lse_gpu=ls, what=f"ramped keys causal={causal}")
    q3, k3 = q.clone(), k.clone()
    q3[:, :, 0] = 4.0
    k3[:, S - 40, 0] = 60.0  # score +240 (x 0.3 scale: ~104 binades) for every query that sees it
    o, ls = run(q3, k3, v, causal, scale=0.3, lse=True)
    compare_attn(o, q3, k3, v, 0.3, causal, lse_gpu=ls, what=f"one dominant key causal={causal}")


def test_heads_past_4_gib():
    """2^17 heads of 256 queries and keys, d = 128, BF16, causal: 8 GiB per tensor, so
    head offsets pass 2^32 bytes. Heads at the start, around 2^15 and 2^16, at the end and
    32 seeded random heads against the oracle; on every head, the first query (which sees
    only key 0) returns v_0 exactly and nothing is NaN."""
    BH, S, d = 1 << 17, 256, 128
    if torch.cuda.mem_get_info()[0] < (40 << 30):
        pytest.skip("needs 40 GiB of free device memory")
    g = torch.Generator(device=DEV).manual_seed(2026)

    def make():
        t = torch.empty(BH, S, d, dtype=torch.bfloat16, device=DEV)
        for h in range(0, BH, 1 << 14):
            t[h:h + (1 << 14)] = torch.randn(1 << 14, S, d, generator=g, device=DEV).to(torch.bfloat16)
        return t

    q, k, v = make(), make(), make()
    o = torch.full_like(q, float("nan"))
    ls = torch.full((BH * S,), float("nan"), device=DEV)
    sm.attention(q, k, v, causal=True, out=o, lse=ls)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2026)
    heads = sorted({0, 1, 2, (1 << 15) - 1, 1 << 15, (1 << 16) - 1, 1 << 16, (1 << 16) + 1,
                    BH - 2, BH - 1, *rng.integers(0, BH, size=32).tolist()})
    idx = torch.tensor(heads, device=DEV)
    st = compare_attn(o[idx], q[idx].cpu(), k[idx].cpu(), v[idx].cpu(), 1.0 / math.sqrt(d), True,
                      lse_gpu=ls.view(BH, S)[idx], what=f"{BH} heads x {S}, {len(heads)} heads")
    log(f"[attn] {BH} heads past 4 GiB, {len(heads)} heads against the oracle: {st}")
    for h in range(0, BH, 1 << 14):
        oc = o[h:h + (1 << 14)]
        assert not torch.isnan(oc).any(), h
        assert torch.equal(oc[:, 0].view(torch.int16), v[h:h + (1 << 14), 0].view(torch.int16)), h
    assert not torch.isnan(ls).any()
