"""GPU parity of the softmax backward (sm_softmax_bwd) against the FP64 oracle: every plan,
widths 1 ... 20000, three dtypes, misaligned and phase-shifted dy/dx, in place, NaN rows,
every kernel instance, the forward -> backward chain on device, caller workspace."""
import math

import numpy as np
import pytest
import torch

import memory_bound_row_sm_amd as sm
import workloads
from parity import compare, compare_bwd, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
PLANS = {"auto": 0, "resident": 1, "persistent": 2, "wide": 3, "split": 4}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sm.lib()


def inputs(M, N, dt, seed):
    """y: a softmax output (computed on the CPU, stored in dt); dy ~ N(0,1) in dt."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, N, generator=g, dtype=torch.float64) * 3
    y = torch.softmax(x, -1).to(TDT[dt])
    dy = torch.randn(M, N, generator=g, dtype=torch.float64).to(TDT[dt])
    return y, dy


def run_bwd(y, dy, plan="auto", dx=None, **kw):
    if dx is None:
        dx = torch.full_like(y, float("nan"))
    sm.softmax_backward(y, dy, dx=dx, opts={"plan": PLANS[plan], **kw})
    torch.cuda.synchronize()
    return dx


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [1, 7, 64, 127, 781, 1000, 2047, 4096, 8192, 8193, 20000])
def test_widths_all_plans(dt, N):
    M = 21 if N <= 8192 else 4
    y, dy = inputs(M, N, dt, seed=N)
    yd, dyd = y.to(DEV), dy.to(DEV)
    for plan in ["auto", "resident", "persistent", "wide", "split"]:
        if plan in ("resident", "persistent") and N > 8192:
            continue
        g = run_bwd(yd, dyd, plan)
        compare_bwd(g, y, dy, what=f"bwd {dt} {M}x{N} {plan}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_phase_shifted_and_strided(dt, plan):
    for N, sy, sd, sx, oy, od, ox in [(100, 103, 100, 100, 1, 0, 3), (1000, 1001, 1003, 1000, 0, 1, 1),
                                      (4097, 4099, 4097, 4101, 3, 0, 0), (9001, 9001, 9005, 9011, 1, 1, 2)]:
        if plan in ("resident", "persistent") and N > 8192:
            continue
        M = 13
        y, dy = inputs(M, N, dt, seed=N + 1)
        by = torch.zeros(M * sy + oy, dtype=TDT[dt], device=DEV)
        bd = torch.zeros(M * sd + od, dtype=TDT[dt], device=DEV)
        bx = torch.full((M * sx + ox + 8,), float("nan"), dtype=TDT[dt], device=DEV)
        yv = by[oy:oy + M * sy].view(M, sy)[:, :N]
        dv = bd[od:od + M * sd].view(M, sd)[:, :N]
        xv = bx[ox:ox + M * sx].view(M, sx)[:, :N]
        yv.copy_(y.to(DEV))
        dv.copy_(dy.to(DEV))
        run_bwd(yv, dv, plan, dx=xv)
        compare_bwd(xv, y, dy, what=f"bwd {dt} N={N} offs={oy},{od},{ox} {plan}")
        assert torch.isnan(bx[ox:ox + M * sx].view(M, sx)[:, N:].float()).all()
        assert torch.isnan(bx[ox + M * sx:].float()).all()


@pytest.mark.parametrize("M,N,dt", [(1, 1500, "f16"), (9, 2000, "bf16"), (1001, 1500, "f16"),
                                     (4099, 2000, "bf16"), (2053, 1000, "f32"), (517, 4000, "bf16")])
def test_resident_rows_sharing_lines(M, N, dt):
    """Resident backward rows of 128+ lanes whose stride is not a whole number of
    128-byte lines run in XCD-contiguous order: every row written as the oracle says."""
    y, dy = inputs(M, N, dt, seed=M + N)
    g = run_bwd(y.to(DEV), dy.to(DEV), "resident")
    compare_bwd(g, y, dy, what=f"bwd {dt} {M}x{N} resident, XCD-contiguous order")


@pytest.mark.parametrize("plan", ["resident", "persistent", "wide", "split"])
def test_in_place(plan):
    for M, N in [(33, 4096), (5, 20000)]:
        if plan in ("resident", "persistent") and N > 8192:
            continue
        y, dy = inputs(M, N, "bf16", seed=M)
        yd, dyd = y.to(DEV), dy.to(DEV)
        run_bwd(yd, dyd, plan, dx=dyd)  # dx over dy
        compare_bwd(dyd, y, dy, what=f"bwd in place over dy {plan}")
        yd, dyd = y.to(DEV), dy.to(DEV)
        run_bwd(yd, dyd, plan, dx=yd)   # dx over y
        compare_bwd(yd, y, dy, what=f"bwd in place over y {plan}")


def test_infinite_dy():
    """dy = +inf where y > 0 makes the dot +inf: dx is -inf where y > 0 and dy is finite,
    NaN at the infinite entry (inf - inf) and where y = 0 (0 * -inf) -- on every plan,
    in FP32 as in the FP64 oracle."""
    for plan in ["resident", "persistent", "wide", "split"]:
        y, dy = inputs(3, 3000, "f32", seed=6)
        y[1, 100:200] = 0.0
        dy[1, 17] = math.inf
        g = run_bwd(y.to(DEV), dy.to(DEV), plan).cpu()
        compare_bwd(g, y, dy, what=f"bwd +inf {plan}")
        assert torch.isinf(g[1]).sum() > 0 and torch.isfinite(g[0]).all()


def test_nan_rows():
    for plan in ["resident", "wide", "split"]:
        y, dy = inputs(3, 3000, "f32", seed=5)
        dy[1, 17] = math.nan
        g = run_bwd(y.to(DEV), dy.to(DEV), plan).cpu()
        assert torch.isnan(g[1]).all() and torch.isfinite(g[0]).all() and torch.isfinite(g[2]).all()
        compare_bwd(g, y, dy, what=f"bwd NaN {plan}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_every_instance(dt):
    N = 500 if dt == "f32" else 1000
    M = 11
    y, dy = inputs(M, N + 1, dt, seed=31)
    yv, dv = y[:, :N], dy[:, :N]                       # stride N + 1
    yd, dyd = y.to(DEV)[:, :N], dy.to(DEV)[:, :N]
    n = 0
    for G in (16, 32, 64, 128, 256, 512, 1024):
        for V in (1, 2, 4):
            if G * V < 126:
                continue
            for plan in ("resident", "persistent"):
                for nt in ((-1, 1) if G >= 128 else (-1,)):
                    info = sm.plan_for_backward(yd, dyd, opts={"plan": PLANS[plan], "lanes_per_row": G,
                                                               "vecs_per_lane": V, "nontemporal": nt})
                    assert info["nt_loads"] == (1 if nt == 1 else 0)
                    g = run_bwd(yd, dyd, plan, lanes_per_row=G, vecs_per_lane=V, grid=5, nontemporal=nt)
                    compare_bwd(g, yv.contiguous(), dv.contiguous(),
                                what=f"bwd {dt} G={G} V={V} {plan} nt={nt}")
                    n += 1
    log(f"[bwd] {dt}: {n} instances")
    assert n >= 50


def test_forward_backward_chain_on_device():
    """The workload's forward output feeds the backward: 4096 x 4096 BF16."""
    x = workloads.normal_bf16_4096x4096(M=1024)
    y = sm.softmax(x.to(DEV))
    dy = torch.randn(1024, 4096, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    g = run_bwd(y, dy.to(DEV))
    st = compare_bwd(g, y.cpu(), dy, what="fwd->bwd chain")
    log(f"[bwd] chain: {st}")
    # and against torch autograd in float32 on the same x (a looser, independent check)
    xt = x.float().requires_grad_(True)
    torch.softmax(xt, -1).backward(dy.float())
    assert float((g.float().cpu() - xt.grad).abs().max()) < 2e-2


@pytest.mark.parametrize("plan", ["wide", "split"])
def test_caller_workspace_and_errors(plan):
    y, dy = inputs(6, 30000, "bf16", seed=9)
    yd, dyd = y.to(DEV), dy.to(DEV)
    opts = {"plan": PLANS[plan]}
    info = sm.plan_for_backward(yd, dyd, opts=opts)
    assert info["plan_name"] == plan
    ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device=DEV)
    for _ in range(2):
        dx = torch.full_like(yd, float("nan"))
        sm.softmax_backward(yd, dyd, dx=dx, opts=opts, workspace=ws)
        torch.cuda.synchronize()
        compare_bwd(dx, y, dy, what=f"bwd caller workspace {plan}")
    with pytest.raises(sm.SoftmaxError) as e:
        sm.softmax_backward(yd, dyd, dx=dx, opts=opts, workspace=ws[:-16])
    assert e.value.status == -6
