"""Calls captured into a HIP graph and replayed with new inputs.

A SPLIT call tags its slots with an id fixed at launch; a graph would replay that id
unchanged, and a replay could then read the previous replay's row statistics. Under
capture the library therefore takes the two-pass WIDE plan for rows that AUTO would
split (RMSNorm: its two-launch form) and refuses a forced SPLIT (SM_ERR_PLAN). Each
replay below runs on a new seeded input, with eager calls and synchronisations
between replays, and is checked against the FP64 oracle."""
import pytest
import torch

import memory_bound_row_sm_amd as sm
from parity import compare, compare_bwd, compare_rms, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    sm.lib()


def _rand(M, N, dt, seed, scale=3.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(M, N, generator=g) * scale).to(dt)


@pytest.mark.parametrize("workspace", [False, True])
@pytest.mark.parametrize("M,N,dt", [(16, 65536, torch.bfloat16), (4, 20000, torch.float32)])
def test_softmax_replays(M, N, dt, workspace):
    xs = torch.empty(M, N, dtype=dt, device=DEV)
    ys = torch.empty_like(xs)
    eager_plan = sm.plan_for(xs, ys)["plan_name"]
    assert eager_plan == "split"
    ws = None
    if workspace:  # caller scratch for either plan (eager SPLIT, captured WIDE)
        nbytes = max(sm.plan_for(xs, ys, opts={"plan": p})["workspace_bytes"]
                     for p in (sm.SM_PLAN_WIDE, sm.SM_PLAN_SPLIT))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    xs.copy_(_rand(M, N, dt, seed=1).to(DEV))
    sm.softmax(xs, out=ys, workspace=ws)  # eager warm-up on the same buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sm.softmax(xs, out=ys, workspace=ws)
        s = torch.cuda.current_stream().cuda_stream
        code = {torch.float32: sm.SM_F32, torch.bfloat16: sm.SM_BF16}[dt]
        rc = sm.sm_softmax_fwd_ex(xs.data_ptr(), ys.data_ptr(), M, N, N, N, code,
                                  {"plan": sm.SM_PLAN_SPLIT}, 0, 0, s)
        assert rc == -7  # a forced SPLIT is refused under capture
    for i in range(REPLAYS):
        x = _rand(M, N, dt, seed=100 + i)
        xs.copy_(x.to(DEV))
        ys.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(ys, x, what=f"replay {i} {M}x{N} {dt} workspace={workspace}")
        e = sm.softmax(xs)  # eager SPLIT call between replays, same input
        torch.cuda.synchronize()
        compare(e, x, what=f"eager after replay {i}")
    log(f"[graph] softmax {M}x{N} {dt} workspace={workspace}: {REPLAYS} replays match the oracle")


def test_backward_replays():
    M, N = 16, 65536
    ys = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    dys, dxs = torch.empty_like(ys), torch.empty_like(ys)
    assert sm.plan_for_backward(ys, dys)["plan_name"] == "split"
    sm.softmax_backward(ys.fill_(0), dys.fill_(0), dx=dxs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sm.softmax_backward(ys, dys, dx=dxs)
    for i in range(REPLAYS):
        y = torch.softmax(_rand(M, N, torch.float32, seed=200 + i).double(), -1).to(torch.bfloat16)
        dy = _rand(M, N, torch.bfloat16, seed=300 + i, scale=1.0)
        ys.copy_(y.to(DEV))
        dys.copy_(dy.to(DEV))
        dxs.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_bwd(dxs, y, dy, what=f"backward replay {i}")


@pytest.mark.parametrize("M,N", [(16, 1 << 18), (4, 1 << 22)])
def test_rmsnorm_replays(M, N):
    xs = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    rs, ys, ss = (torch.empty_like(xs) for _ in range(3))
    wv = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    info = sm.plan_for_rmsnorm(xs, wv, residual=rs)
    # one-launch SPLIT eagerly (two launches under capture), or already the two-launch form
    # on rows of more than 256 slices, whose second launch sums each row once per workgroup
    assert info["plan_name"] == ("wide" if N >= 1 << 22 else "split"), info
    assert N < 1 << 22 or info["waves_per_row"] > 256
    sm.rmsnorm(xs.fill_(1), wv.fill_(1), residual=rs.fill_(0), out=ys, residual_out=ss)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sm.rmsnorm(xs, wv, residual=rs, out=ys, residual_out=ss)
    for i in range(REPLAYS):
        gen = torch.Generator().manual_seed(400 + i)
        x = (torch.randn(M, N, generator=gen) * 2).to(torch.bfloat16)
        r = torch.randn(M, N, generator=gen).to(torch.bfloat16)
        w = (1 + 0.5 * torch.randn(N, generator=gen)).to(torch.bfloat16)
        xs.copy_(x.to(DEV))
        rs.copy_(r.to(DEV))
        wv.copy_(w.to(DEV))
        ys.fill_(float("nan"))
        ss.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_rms(ys, x, r, w, 1e-6, s_gpu=ss, what=f"rmsnorm replay {i}")
