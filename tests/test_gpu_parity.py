"""GPU parity: the HIP library against the FP64 oracle, element by element, on the
seeded workloads at full size (the 2 GiB attention-shaped case block by block), on
every plan, on ragged, misaligned, strided and in-place layouts, and on the special
values.

Every output buffer is filled with NaN before the kernel runs, so a skipped
store cannot hide behind stale values ("Measured optimization case studies",
section "CUDA: parallel reduction, online statistics and a numerical fix").
"""
import math

import numpy as np
import pytest
import torch

import memory_bound_row_sm_amd as sm
import oracle
import workloads
from parity import compare, compare_bwd, log, row_sum_bound, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
PLANS = {"auto": sm.SM_PLAN_AUTO, "resident": sm.SM_PLAN_RESIDENT,
         "persistent": sm.SM_PLAN_PERSISTENT, "wide": sm.SM_PLAN_WIDE, "split": sm.SM_PLAN_SPLIT}


def run(x_dev, plan="auto", out=None, **kw):
    """Softmax through the C ABI with a NaN-prefilled output; synchronises."""
    if out is None:
        out = torch.full_like(x_dev, float("nan"))
    opts = {"plan": PLANS[plan], **kw}
    sm.softmax(x_dev, out=out, opts=opts)
    torch.cuda.synchronize()
    return out


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    sm.lib()


# ------------------------------------------------------------------ workloads, full size

SMALL_WORKLOADS = ["normal_f32_128x781", "normal_bf16_4096x4096",
                   *[f"spiky_f16_8192x{n}" for n in workloads.SPIKE_WIDTHS],
                   "offset_bf16_64x131072"]


@pytest.mark.parametrize("name", SMALL_WORKLOADS)
def test_workload_full_auto_plan(name):
    x = workloads.generate(name)
    log(f"[parity] {name} auto plan, shape {tuple(x.shape)} {x.dtype}")
    xd = x.to(DEV)
    info = sm.plan_for(xd)
    g = run(xd)
    st = compare(g, x, what=name)
    log(f"[parity] {name}: plan={info['plan_name']} G={info['lanes_per_row']} "
        f"V={info['vecs_per_lane']} {st}")
    sums = g.double().sum(dim=1).cpu().numpy()
    assert np.max(np.abs(sums - 1)) <= row_sum_bound(workloads.dtype_name(x))


@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
@pytest.mark.parametrize("name", ["normal_f32_128x781", "normal_bf16_4096x4096",
                                  "spiky_f16_8192x127", "spiky_f16_8192x1000",
                                  "spiky_f16_8192x8192", "offset_bf16_64x131072"])
def test_workload_forced_plans(name, plan):
    x = workloads.generate(name)
    if plan in ("resident", "persistent") and x.shape[1] > 8192:
        x = x[:, :32768].contiguous()  # one-pass plans hold at most 1024 x 8 windows per row
    log(f"[parity] {name} plan={plan} shape {tuple(x.shape)}")
    g = run(x.to(DEV), plan)
    st = compare(g, x, what=f"{name}/{plan}")
    log(f"[parity] {name}/{plan}: {st}")


CAUSAL_BLOCK = 16384  # rows per oracle comparison block (32 blocks of 64 MiB)


@pytest.fixture(scope="module")
def causal_full():
    """524288 x 2048 BF16 causal logits (8 x 32 heads of 2048 x 2048), their softmax
    in the bench's automatic launch configuration, and that output's backward with a
    seeded dy, all resident on the GPU; the host copy of the input for the oracle."""
    log("[parity] causal_bf16_524288x2048: generating (CPU) ...")
    x = workloads.generate("causal_bf16_524288x2048")
    xd = x.to(DEV)
    info = sm.plan_for(xd)
    log(f"[parity] causal plan {info['plan_name']} G={info['lanes_per_row']} "
        f"V={info['vecs_per_lane']} nt={info['nt_loads']}: running on GPU")
    g = run(xd)
    del xd
    dy = workloads.upstream_grad(g.shape, "bf16", device=DEV)
    binfo = sm.plan_for_backward(g, dy)
    log(f"[parity] causal backward plan {binfo['plan_name']} G={binfo['lanes_per_row']} "
        f"V={binfo['vecs_per_lane']} nt={binfo['nt_loads']}")
    dx = torch.full_like(g, float("nan"))
    sm.softmax_backward(g, dy, dx=dx)
    torch.cuda.synchronize()
    yield x, g, dy, dx
    del g, dy, dx
    torch.cuda.empty_cache()


CAUSAL_PARTS = 4  # each test compares a quarter of the rows (8 blocks)


def _causal_rows(part, M):
    per = M // CAUSAL_PARTS
    return range(part * per, M if part == CAUSAL_PARTS - 1 else (part + 1) * per, CAUSAL_BLOCK)


@pytest.mark.parametrize("part", range(CAUSAL_PARTS))
def test_causal_logits_full_size(causal_full, part):
    """Every row of the 524288 x 2048 output against the oracle, block by block (the
    element-wise gates on every element of the config; a quarter of the rows per
    test)."""
    x, g, _, _ = causal_full
    M = x.shape[0]
    worst = {"worst_frac_of_tol": 0.0, "max_ulp_vs_rounded": 0.0, "max_rel_thr": 0.0}
    blocks = _causal_rows(part, M)
    for r0 in blocks:
        r1 = min(M, r0 + CAUSAL_BLOCK)
        st = compare(g[r0:r1].cpu(), x[r0:r1], what=f"causal rows {r0}:{r1}")
        for k in worst:
            worst[k] = max(worst[k], st[k])
    log(f"[parity] causal rows {blocks.start}:{min(M, blocks.stop)} compared; worst {worst}")


def test_causal_logits_properties(causal_full):
    """What the causal mask fixes, on every row: masked keys exactly 0, the first
    query of each head one-hot, rows summing to 1 within the BF16 bound."""
    x, g, _, _ = causal_full
    M = x.shape[0]
    Q = 2048
    heads = M // Q
    i = torch.arange(Q, device=DEV)
    masked = (i[None, :] > i[:, None])
    gv = g.view(heads, Q, Q)
    assert not torch.isnan(gv).any()
    assert (gv.masked_select(masked.expand_as(gv)) == 0).all()
    assert (gv[:, 0, 0] == 1).all()
    sums = gv.sum(dim=-1, dtype=torch.float64)
    assert float((sums - 1).abs().max()) <= row_sum_bound("bf16")


@pytest.mark.parametrize("part", range(CAUSAL_PARTS))
def test_causal_logits_backward_full_size(causal_full, part):
    """The backward of the same 524288 x 2048 output, every row against the oracle
    block by block (a quarter of the rows per test)."""
    _, g, dy, dx = causal_full
    M = g.shape[0]
    worst = 0.0
    blocks = _causal_rows(part, M)
    for r0 in blocks:
        r1 = min(M, r0 + CAUSAL_BLOCK)
        st = compare_bwd(dx[r0:r1].cpu(), g[r0:r1].cpu(), dy[r0:r1].cpu(),
                         what=f"causal backward rows {r0}:{r1}")
        worst = max(worst, st["worst_frac_of_tol"])
    log(f"[parity] causal backward rows {blocks.start}:{min(M, blocks.stop)} compared; "
        f"worst fraction of tolerance {worst}")


def test_causal_logits_backward_properties(causal_full):
    """dx is exactly 0 where y is, and each row of dx sums to about 0."""
    _, g, dy, dx = causal_full
    M = g.shape[0]
    Q = 2048
    heads = M // Q
    i = torch.arange(Q, device=DEV)
    masked = (i[None, :] > i[:, None])
    dv = dx.view(heads, Q, Q)
    assert not torch.isnan(dv).any()
    assert (dv.masked_select(masked.expand_as(dv)) == 0).all()  # y = 0 there
    assert float(dv.sum(dim=-1, dtype=torch.float64).abs().max()) < 0.05  # d (1 - sum y)


# ------------------------------------------------------------------ shapes and layouts

def _rand(M, N, dt, seed, scale=3.0):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal((M, N)) * scale).astype(np.float32)).to(TDT[dt])


WIDTHS = [1, 2, 7, 8, 9, 63, 64, 65, 127, 129, 255, 781, 1000, 1023, 1025, 2047, 4095, 4097,
          6272, 8191, 8192, 8193, 16381, 32769]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", WIDTHS)
def test_width_grid_all_plans(dt, N):
    M = 37 if N <= 8192 else 5
    x = _rand(M, N, dt, seed=N)
    xd = x.to(DEV)
    for plan in ["auto", "resident", "persistent", "wide", "split"]:
        if plan in ("resident", "persistent") and N > 8192 and dt == "f32" and N > 16384:
            continue
        g = run(xd, plan)
        compare(g, x, what=f"{dt} {M}x{N} {plan}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_misaligned_strided_and_phase_shifted(dt, plan):
    """Base pointers off by one element, row strides that break 16-byte alignment,
    and an output whose 16-byte phase differs from the input's."""
    for N, stride_in, stride_out, off_in, off_out in [
        (100, 103, 100, 1, 1), (100, 100, 107, 0, 3), (1000, 1001, 1003, 1, 2),
        (4097, 4099, 4097, 3, 0), (9000, 9011, 9001, 1, 1)]:
        M = 23
        base = _rand(M * stride_in + off_in, 1, dt, seed=N).view(-1)
        xin = base[off_in:off_in + M * stride_in].view(M, stride_in)[:, :N]
        ob = torch.full((M * stride_out + off_out + 8,), float("nan"), dtype=TDT[dt], device=DEV)
        out = ob[off_out:off_out + M * stride_out].view(M, stride_out)[:, :N]
        xd = base.to(DEV)[off_in:off_in + M * stride_in].view(M, stride_in)[:, :N]
        if plan in ("resident", "persistent") and N > 8192 and dt == "f32":
            continue
        run(xd, plan, out=out)
        compare(out, xin.contiguous(), what=f"{dt} {N} si={stride_in} so={stride_out} "
                                            f"offs={off_in},{off_out} {plan}")
        # untouched: the gaps between rows and the guard elements after the last row
        gaps = ob[off_out:off_out + M * stride_out].view(M, stride_out)[:, N:]
        assert torch.isnan(gaps.float()).all()
        assert torch.isnan(ob[:off_out].float()).all()
        assert torch.isnan(ob[off_out + M * stride_out:].float()).all()


@pytest.mark.parametrize("M,N,dt", [(1, 1500, "f16"), (7, 1500, "f16"), (8, 2000, "bf16"),
                                     (9, 2000, "bf16"), (1001, 1500, "f16"), (4099, 2000, "bf16"),
                                     (2053, 1000, "f32"), (517, 4000, "bf16"), (300, 1000, "f16")])
def test_resident_rows_sharing_lines(M, N, dt):
    """Resident rows of 128+ lanes whose stride is not a whole number of 128-byte
    lines run in XCD-contiguous order (the workgroups renumbered by a permutation;
    the last case, 64-lane rows, keeps the hardware's order): every row,
    row group and grid size (multiple of the XCD count or not) is written exactly as
    the oracle says, and nothing else is."""
    x = _rand(M, N, dt, seed=M + N)
    g = run(x.to(DEV), "resident")
    compare(g, x, what=f"{dt} {M}x{N} resident, XCD-contiguous order")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_in_place(dt, plan):
    for M, N in [(64, 781), (33, 4096), (5, 20000)]:
        if plan in ("resident", "persistent") and N > 8192:
            continue
        x = _rand(M, N, dt, seed=M)
        xd = x.to(DEV)
        run(xd, plan, out=xd)
        compare(xd, x, what=f"in place {dt} {M}x{N} {plan}")


def test_canaries_around_output():
    for plan in ["resident", "persistent", "wide", "split"]:
        M, N = 19, 3000
        x = _rand(M, N, "bf16", seed=3)
        buf = torch.full((M * N + 256,), -7.0, dtype=torch.bfloat16, device=DEV)
        out = buf[128:128 + M * N].view(M, N)
        run(x.to(DEV), plan, out=out)
        compare(out, x, what=f"canary {plan}")
        assert (buf[:128] == -7).all() and (buf[128 + M * N:] == -7).all()


# ------------------------------------------------------------------ special values

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_masked_rows_every_plan(dt, plan):
    """-inf entries give exactly 0, fully masked rows give zeros, and masked prefixes
    wider than a chunk stay NaN-free ("Measured optimization case studies", section
    "Wide rows: loop in one program, or split across programs": masked rows on every
    plan)."""
    N = 12000 if plan in ("wide", "split") else 3000
    x = _rand(6, N, dt, seed=11).float()
    x[0, :] = -math.inf                    # fully masked row
    x[1, : N - 5] = -math.inf              # masked prefix, 5 live entries at the end
    x[2, 5:] = -math.inf                   # 5 live entries at the start
    x[3, ::2] = -math.inf                  # every other entry
    x[4, 1024:3072] = -math.inf            # whole chunks masked in the middle
    x = x.to(TDT[dt])
    g = run(x.to(DEV), plan)
    compare(g, x, what=f"masked {dt} {plan}")
    gc = g.float().cpu()
    assert (gc[0] == 0).all()
    assert (gc[1, : N - 5] == 0).all()


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_nan_and_inf_rows(dt, plan):
    x = _rand(4, 2000, dt, seed=12).float()
    x[0, 17] = math.nan
    x[1, 1999] = math.inf
    x[2, 0] = math.nan
    x[2, 1:] = -math.inf
    x = x.to(TDT[dt])
    g = run(x.to(DEV), plan).float().cpu()
    assert torch.isnan(g[0]).all() and torch.isnan(g[1]).all() and torch.isnan(g[2]).all()
    compare(g[3:4], x[3:4], what=f"row after NaN rows {dt} {plan}")


@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_extreme_magnitudes(plan):
    # BF16 logits near the top of the FP32 range, and FP16 +/-1e4 spikes
    x = torch.zeros(4, 3000)
    x[0, :] = -3.0e38
    x[0, 7] = 3.0e38
    x[1, :] = 3.0e38
    x[2, :] = torch.linspace(-3e38, 3e38, 3000)
    x[3, :] = 1e4
    xb = x.to(torch.bfloat16)
    compare(run(xb.to(DEV), plan), xb, what=f"huge bf16 {plan}")
    xf = x.to(torch.float32)
    compare(run(xf.to(DEV), plan), xf, what=f"huge f32 {plan}")
    s = workloads.spiky_f16(4096, M=64)
    compare(run(s.to(DEV), plan), s, what=f"spikes f16 {plan}")


@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_outputs_near_the_bottom_of_the_range(plan):
    """Probabilities from 1e-30 down past the smallest normal FP32 (2^-126) into the
    BF16 and FP16 subnormals: the one-ulp gate holds (BF16 with its 2^-126 floor,
    where the FP32 exponential flushes), and the FP32 tolerance's 2^-126 floor."""
    N = 3000
    x = torch.zeros(3, N)
    x[:, 1:] = -torch.linspace(60.0, 110.0, N - 1)   # exp(-60) ... exp(-110)
    x[1, 7] = 5.0
    x[2, ::3] = -math.inf
    x[2, 0] = 0.0
    for dt in ("bf16", "f16", "f32"):
        xt = x.to(TDT[dt])
        st = compare(run(xt.to(DEV), plan), xt, what=f"bottom of the range {dt} {plan}")
        log(f"[parity] bottom of the range {dt} {plan}: {st}")


def test_constant_and_single_element_rows():
    for dt in ["f32", "f16", "bf16"]:
        for N in [1, 781, 8192, 10000]:
            x = torch.full((3, N), 1.5).to(TDT[dt])
            g = run(x.to(DEV))
            compare(g, x, what=f"constant {dt} {N}")
            if dt == "f32":  # exp(0) = 1 and the compensated sum is exactly N: y = fl(1/N)
                want = torch.full((3, N), 1.0 / N, dtype=torch.float64).float()
                assert torch.equal(g.cpu(), want), N


# ------------------------------------------------------------------ invariants

def test_bitwise_repeatable_and_plans_agree():
    x = workloads.normal_bf16_4096x4096(M=512).to(DEV)
    a = run(x)
    b = run(x)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for plan in ["resident", "persistent", "wide", "split"]:
        c = run(x, plan)
        d = run(x, plan)
        assert torch.equal(c.view(torch.int16), d.view(torch.int16))
        assert float((c.float() - a.float()).abs().max()) <= 2 * 2.0 ** -8


def test_shift_invariance():
    rng = np.random.default_rng(5)
    xi = rng.integers(-8, 9, size=(64, 1500)).astype(np.float32)
    for dt in ["f32", "bf16"]:
        for plan in ["auto", "split"]:  # SPLIT: slice and row maxima shift alike
            a = run(torch.from_numpy(xi).to(TDT[dt]).to(DEV), plan, vecs_per_lane=1 if plan == "split" else 0)
            b = run(torch.from_numpy(xi + 64).to(TDT[dt]).to(DEV), plan,
                    vecs_per_lane=1 if plan == "split" else 0)
            if dt == "f32":  # x - max is exact on this grid: bitwise equal
                assert torch.equal(a, b), plan
            else:
                assert float((a.float() - b.float()).abs().max()) <= 2.0 ** -8


def test_permutation_equivariance():
    x = _rand(16, 3000, "f32", seed=9).to(DEV)
    perm = torch.randperm(3000, generator=torch.Generator().manual_seed(0)).to(DEV)
    a = run(x)[:, perm]
    b = run(x[:, perm].contiguous())
    assert torch.allclose(a, b, rtol=2e-6, atol=0)


# ------------------------------------------------------------------ API behaviour on device

def test_zero_sized_and_rejected_calls_launch_nothing():
    x = torch.randn(0, 8, device=DEV)
    assert sm.sm_softmax_fwd(x.data_ptr(), x.data_ptr(), 0, 8, 8, 8, sm.SM_F32, 0) == 0
    y = torch.randn(4, 100, device=DEV)
    rc = sm.sm_softmax_fwd_ex(y.data_ptr(), y.data_ptr(), 4, 100, 100, 100, sm.SM_F32,
                              {"plan": sm.SM_PLAN_PERSISTENT, "lanes_per_row": 16,
                               "vecs_per_lane": 1}, 0, 0, 0)
    assert rc == -7  # 16 lanes x 1 vector cannot hold 100 FP32 elements


@pytest.mark.parametrize("plan", ["wide", "split"])
def test_caller_workspace(plan):
    x = _rand(8, 20000, "bf16", seed=4)
    xd = x.to(DEV)
    opts = {"plan": PLANS[plan]}
    info = sm.plan_for(xd, opts=opts)
    assert info["plan_name"] == plan
    ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device=DEV)
    for _ in range(3):  # SPLIT reuses the same slots call after call (new tags each time)
        out = torch.full_like(xd, float("nan"))
        sm.softmax(xd, out=out, opts=opts, workspace=ws)
        torch.cuda.synchronize()
        compare(out, x, what=f"caller workspace {plan}")
    small = torch.empty(info["workspace_bytes"] - 8, dtype=torch.uint8, device=DEV)
    with pytest.raises(sm.SoftmaxError) as e:
        sm.softmax(xd, out=out, opts=opts, workspace=small)
    assert e.value.status == -6


def test_batched_views_through_python_binding():
    x = torch.randn(2, 3, 50, 300, dtype=torch.float16)
    g = sm.softmax(x.to(DEV))
    torch.cuda.synchronize()
    compare(g.view(-1, 300), x.view(-1, 300), what="4-d tensor")


def test_bench_copy_and_flush():
    n = 1 << 22
    a = torch.randint(0, 1 << 30, (n // 4,), dtype=torch.int32, device=DEV)
    for scope in (0, 1):  # plain and device-scope stores
        b = torch.zeros_like(a)
        assert sm.sm_bench_copy(a.data_ptr(), b.data_ptr(), n, 0, scope, 0, None, None) == 0
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    assert sm.sm_bench_copy(a.data_ptr(), b.data_ptr(), n, 0, 2, 0, None, None) == -1  # bad scope
    assert sm.sm_bench_flush(b.data_ptr(), n, 0) == 0
    torch.cuda.synchronize()
    assert torch.equal(b, a)  # the sweep only reads


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_every_row_kernel_instance(dt):
    """Each built (lanes per row, vectors per lane, prefetch) instance, on the resident
    and persistent plans, on ragged rows that start misaligned."""
    es = 4 if dt == "f32" else 2
    N = 500 if dt == "f32" else 1000        # 125 windows of 16 bytes (+1 when misaligned)
    M = 29
    base = _rand(M * (N + 1) + 1, 1, dt, seed=17).view(-1)
    x = base[1:1 + M * (N + 1)].view(M, N + 1)[:, :N]   # stride N + 1, offset one element
    xd = base.to(DEV)[1:1 + M * (N + 1)].view(M, N + 1)[:, :N]
    n = 0
    for G in (16, 32, 64, 128, 256, 512, 1024):
        for V in (1, 2, 4, 8):
            if G * V * 16 < (N + 16 // es) * es:
                continue
            for plan, pf, nt in (("resident", 0, -1), ("resident", 0, 1), ("persistent", 0, -1),
                                 ("persistent", 1, -1)):
                if (pf and G > 256) or (nt == 1 and G < 128):
                    continue
                g = run(xd, plan, lanes_per_row=G, vecs_per_lane=V, prefetch=1 if pf else -1,
                        nontemporal=nt, grid=7)
                compare(g, x.contiguous(), what=f"{dt} G={G} V={V} {plan} pf={pf} nt={nt}")
                n += 1
    for nt in (-1, 1):  # both wide-path instances
        g = run(xd, "wide", nontemporal=nt)
        compare(g, x.contiguous(), what=f"{dt} wide nt={nt}")
    log(f"[parity] {dt}: {n} row-kernel instances checked")
    assert n >= 50
