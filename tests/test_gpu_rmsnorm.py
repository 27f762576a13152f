"""GPU parity of the fused residual RMSNorm (sm_rmsnorm_fwd) against the FP64 oracle:
the pages' shapes, every plan, widths 1 ... 70001, three dtypes, with and without a
residual and residual_out, misaligned and phase-shifted tensors and weight, in place,
special values, every kernel instance, caller workspace."""
import math

import pytest
import torch

import memory_bound_row_sm_amd as sm
from parity import compare_rms, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
PLANS = {"auto": 0, "resident": 1, "persistent": 2, "wide": 3, "split": 4}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    sm.lib()


def inputs(M, N, dt, seed, residual=True):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(M, N, generator=g) * 2).to(TDT[dt])
    r = (torch.randn(M, N, generator=g)).to(TDT[dt]) if residual else None
    w = (1 + 0.5 * torch.randn(N, generator=g)).to(TDT[dt])
    return x, r, w


def run(x, r, w, plan="auto", eps=1e-6, s_out=False, **kw):
    xd, wd = x.to(DEV), w.to(DEV)
    rd = None if r is None else r.to(DEV)
    y = torch.full_like(xd, float("nan"))
    s = torch.full_like(xd, float("nan")) if s_out else None
    sm.rmsnorm(xd, wd, residual=rd, eps=eps, out=y, residual_out=s, opts={"plan": PLANS[plan], **kw})
    torch.cuda.synchronize()
    return y, s


@pytest.mark.parametrize("plan", ["auto", "resident", "persistent", "split", "wide"])
def test_warpline_shapes(plan):
    """Batch x hidden of the Warpline README's K1 table, BF16, residual and residual_out."""
    for M, N in [(1, 1024), (8, 1024), (16, 2048), (32, 4096), (64, 4096), (64, 8192)]:
        x, r, w = inputs(M, N, "bf16", seed=M + N)
        y, s = run(x, r, w, plan, s_out=True)
        st = compare_rms(y, x, r, w, 1e-6, s_gpu=s, what=f"K1 {M}x{N} {plan}")
        assert st["worst_frac_of_tol"] <= 1.0


def test_case_study_shapes_auto():
    """The FP16 shapes of "Measured optimization case studies" (residual RMSNorm)."""
    for M, N in [(32, 127), (1024, 1024), (512, 4097), (16384, 4096), (4, 32769), (64, 131072)]:
        x, r, w = inputs(M, N, "f16", seed=N)
        info = sm.plan_for_rmsnorm(x.to(DEV), w.to(DEV), residual=r.to(DEV))
        y, s = run(x, r, w, s_out=True)
        st = compare_rms(y, x, r, w, 1e-6, s_gpu=s, what=f"case study {M}x{N}")
        log(f"[rms] {M}x{N}: plan {info['plan_name']} V={info['vecs_per_lane']} "
            f"P={info['waves_per_row']}: {st}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 7, 64, 127, 781, 1000, 2047, 4096, 8192, 8193, 20000, 70001])
def test_widths_all_plans(dt, N):
    M = 21 if N <= 8192 else 4
    for residual in (True, False):
        x, r, w = inputs(M, N, dt, seed=N, residual=residual)
        for plan in ["auto", "resident", "persistent", "split", "wide"]:
            if plan in ("resident", "persistent") and N > 16384:
                continue
            y, s = run(x, r, w, plan, eps=1e-5, s_out=residual)
            compare_rms(y, x, r, w, 1e-5, s_gpu=s, what=f"{dt} {M}x{N} {plan} res={residual}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("plan", ["resident", "persistent", "split", "wide"])
def test_misaligned_and_phase_shifted(dt, plan):
    for N, ox, orr, oy, os_, ow in [(100, 1, 0, 3, 2, 1), (1000, 0, 3, 1, 0, 5), (4097, 3, 1, 0, 1, 2),
                                    (9001, 1, 2, 3, 0, 0)]:
        if plan in ("resident", "persistent") and N > 8192:
            continue
        M = 13
        x, r, w = inputs(M, N, dt, seed=N)
        def buf(t, off, fill=0.0):
            b = torch.full((M * N + off + 8,), fill, dtype=TDT[dt], device=DEV)
            v = b[off:off + M * N].view(M, N)
            if t is not None:
                v.copy_(t.to(DEV))
            return b, v
        _, xv = buf(x, ox)
        _, rv = buf(r, orr)
        yb, yv = buf(None, oy, float("nan"))
        sb, sv = buf(None, os_, float("nan"))
        wb = torch.zeros(N + ow + 8, dtype=TDT[dt], device=DEV)
        wv = wb[ow:ow + N]
        wv.copy_(w.to(DEV))
        sm.rmsnorm(xv, wv, residual=rv, eps=1e-6, out=yv, residual_out=sv, opts={"plan": PLANS[plan]})
        torch.cuda.synchronize()
        compare_rms(yv, x, r, w, 1e-6, s_gpu=sv, what=f"{dt} N={N} offs={ox},{orr},{oy},{os_},{ow} {plan}")
        assert torch.isnan(yb[:oy].float()).all() and torch.isnan(yb[oy + M * N:].float()).all()
        assert torch.isnan(sb[:os_].float()).all() and torch.isnan(sb[os_ + M * N:].float()).all()


@pytest.mark.parametrize("plan", ["resident", "split", "wide"])
def test_in_place(plan):
    for M, N in [(33, 4096), (5, 20000)]:
        if plan == "resident" and N > 8192:
            continue
        x, r, w = inputs(M, N, "bf16", seed=M)
        wd = w.to(DEV)
        # y over x, residual_out over the residual (the usual fused-layer update)
        xd, rd = x.to(DEV), r.to(DEV)
        sm.rmsnorm(xd, wd, residual=rd, out=xd, residual_out=rd, opts={"plan": PLANS[plan]})
        torch.cuda.synchronize()
        compare_rms(xd, x, r, w, 1e-6, s_gpu=rd, what=f"in place y=x s=r {plan}")
        # y over the residual, residual_out over x
        xd, rd = x.to(DEV), r.to(DEV)
        sm.rmsnorm(xd, wd, residual=rd, out=rd, residual_out=xd, opts={"plan": PLANS[plan]})
        torch.cuda.synchronize()
        compare_rms(rd, x, r, w, 1e-6, s_gpu=xd, what=f"in place y=r s=x {plan}")


@pytest.mark.parametrize("plan", ["resident", "split", "wide"])
def test_special_values(plan):
    x, r, w = inputs(5, 3000, "f32", seed=4)
    x[0] = 0.0
    r[0] = 0.0
    x[1, 17] = math.nan
    x[2, 5] = math.inf
    for eps in (0.0, 1e-6):
        y, _ = run(x, r, w, plan, eps=eps)
        compare_rms(y, x, r, w, eps, what=f"special eps={eps} {plan}")
        yc = y.cpu()
        assert torch.isnan(yc[1]).all()
        assert torch.isnan(yc[0]).all() if eps == 0.0 else (yc[0] == 0).all()


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_every_instance(dt):
    N = 500 if dt == "f32" else 1000
    x, r, w = inputs(11, N, dt, seed=31)
    n = 0
    for G in (16, 32, 64, 128, 256, 512, 1024):
        for V in (1, 2, 4):
            if G * V < 126:
                continue
            for plan in ("resident", "persistent"):
                for nt in ((-1, 1) if G >= 128 else (-1,)):
                    y, s = run(x, r, w, plan, s_out=True, lanes_per_row=G, vecs_per_lane=V, grid=5,
                               nontemporal=nt)
                    compare_rms(y, x, r, w, 1e-6, s_gpu=s, what=f"{dt} G={G} V={V} {plan} nt={nt}")
                    n += 1
    for V in (1, 2, 4):
        for plan in ("split", "wide"):
            for nt in (-1, 1):
                xx, rr, ww = inputs(3, 40000, dt, seed=V)
                y, s = run(xx, rr, ww, plan, s_out=True, vecs_per_lane=V, nontemporal=nt)
                compare_rms(y, xx, rr, ww, 1e-6, s_gpu=s, what=f"{dt} V={V} {plan} nt={nt}")
                n += 1
    log(f"[rms] {dt}: {n} instances")


def test_rounds_repeatable_and_workspace():
    before = sm.sync_failures()  # cumulative per stream
    x, r, w = inputs(13, 20000, "bf16", seed=5)
    xd, rd, wd = x.to(DEV), r.to(DEV), w.to(DEV)
    P = sm.plan_for_rmsnorm(xd, wd, residual=rd, opts={"plan": 4, "vecs_per_lane": 1})["waves_per_row"]
    y, _ = run(x, r, w, "split", vecs_per_lane=1, grid=P)
    compare_rms(y, x, r, w, 1e-6, what="split rounds")
    a, _ = run(x, r, w)
    b, _ = run(x, r, w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for plan in ("split", "wide"):
        info = sm.plan_for_rmsnorm(xd, wd, residual=rd, opts={"plan": PLANS[plan]})
        ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device=DEV)
        for _ in range(2):
            out = torch.full_like(xd, float("nan"))
            sm.rmsnorm(xd, wd, residual=rd, out=out, opts={"plan": PLANS[plan]}, workspace=ws)
            torch.cuda.synchronize()
            compare_rms(out, x, r, w, 1e-6, what=f"workspace {plan}")
        with pytest.raises(sm.SoftmaxError) as e:
            sm.rmsnorm(xd, wd, residual=rd, out=out, opts={"plan": PLANS[plan]}, workspace=ws[:-16])
        assert e.value.status == -6
    assert sm.sync_failures() == before


def test_against_torch_rms_norm():
    """An independent check in FP32: torch's rms_norm of the rounded sum."""
    x, r, w = inputs(64, 4096, "bf16", seed=9)
    y, s = run(x, r, w, s_out=True)
    st = (x.float() + r.float()).to(torch.bfloat16)
    assert torch.equal(s.cpu().view(torch.int16), st.view(torch.int16))
    want = torch.nn.functional.rms_norm(st.float(), (4096,), weight=w.float(), eps=1e-6)
    assert float((y.float().cpu() - want).abs().max()) <= 2 ** -7 * float(want.abs().max())


@pytest.mark.parametrize("M", [1, 8])
def test_widest_rows_automatic_launch_count(M):
    """Width 2^20 (FP16): one row fits one round of resident slices (one fused launch);
    eight rows need several rounds of more than 64 slices each, where the automatic plan
    takes the two-launch form (publish, then gather and apply) — both against the oracle,
    with a residual and residual_out."""
    N = 1 << 20
    x, r, w = inputs(M, N, "f16", seed=M + 17)
    info = sm.plan_for_rmsnorm(x.to(DEV), w.to(DEV), residual=r.to(DEV))
    log(f"[rms] {M}x{N}: plan {info['plan_name']} launches {info['launches']} "
        f"P={info['waves_per_row']} grid={info['grid']}")
    assert info["launches"] == (2 if M == 8 else 1)
    y, s = run(x, r, w, s_out=True)
    compare_rms(y, x, r, w, 1e-6, s_gpu=s, what=f"widest {M}x{N}")


@pytest.mark.parametrize("dt,M,N", [("bf16", 4, 1 << 22), ("f32", 3, 1 << 21), ("f16", 2, (1 << 22) + 12345)])
def test_two_launch_rows_of_many_slices(dt, M, N):
    """Rows of more than 256 slices in the two-launch form: the second launch sums each
    row's published partials once per workgroup with all its lanes (a fixed tree, so
    every slice applies bitwise the same total); against the oracle with a residual and
    residual_out, and repeatable bit for bit."""
    x, r, w = inputs(M, N, dt, seed=N % 1000 + M)
    info = sm.plan_for_rmsnorm(x.to(DEV), w.to(DEV), residual=r.to(DEV))
    log(f"[rms] {dt} {M}x{N}: plan {info['plan_name']} launches {info['launches']} "
        f"P={info['waves_per_row']} grid={info['grid']}")
    assert info["launches"] == 2 and info["waves_per_row"] > 256
    y, s = run(x, r, w, s_out=True)
    st = compare_rms(y, x, r, w, 1e-6, s_gpu=s, what=f"two launches {dt} {M}x{N}")
    log(f"[rms] {dt} {M}x{N}: {st}")
    y2, _ = run(x, r, w, s_out=True)
    assert torch.equal(y.view(torch.uint8), y2.view(torch.uint8))


def test_split_wait_budget_runs_out():
    """The one-launch SPLIT form with a one-poll wait budget (forced from the host):
    slices that give up count the failure and, since neither output aliases x or the
    residual, form the row's sum of squares from x + r themselves: oracle parity,
    residual_out bit-exact. In place over x they write NaN over their slice instead."""
    M, N = 24, 131072
    x, r, w = inputs(M, N, "bf16", seed=41)
    before = sm.sync_failures()
    y, s = run(x, r, w, "split", s_out=True, vecs_per_lane=1, spin_limit=1)
    n = sm.sync_failures() - before
    compare_rms(y, x, r, w, 1e-6, s_gpu=s, what="one-poll budget, out of place")
    log(f"[rms] one-poll budget: {n} slices fell back to the whole row")
    assert n > 0
    xd, rd, wd = x.to(DEV), r.to(DEV), w.to(DEV)
    before = sm.sync_failures()
    sm.rmsnorm(xd, wd, residual=rd, out=xd, opts={"plan": PLANS["split"], "vecs_per_lane": 1,
                                                   "spin_limit": 1})
    torch.cuda.synchronize()
    n = sm.sync_failures() - before
    P = sm.plan_for_rmsnorm(xd, wd, residual=rd, opts={"plan": PLANS["split"],
                                                        "vecs_per_lane": 1})["waves_per_row"]
    gc = xd.float().cpu().view(M, P, -1)
    nan_slices = torch.isnan(gc).all(dim=2)
    assert not (torch.isnan(gc).any(dim=2) & ~nan_slices).any()
    assert n == int(nan_slices.sum())
    ok_rows = [i for i in range(M) if not nan_slices[i].any()]
    if ok_rows:
        compare_rms(xd[ok_rows], x[ok_rows], r[ok_rows], w, 1e-6, what="in place: rows without timeouts")
