"""GPU tests of the one-launch SPLIT plan (forward and backward): every slice shape,
rounds (more row slices than the grid), rows whose slices are fully masked, the
wait budget (its whole-row fallback out of place, NaN slices in place) and its
failure count, caller workspace, two streams at once, and the bench's wide-row
workload at full size. Each result is checked against the FP64
oracle element by element."""
import math

import pytest
import torch

import memory_bound_row_sm_amd as sm
import workloads
from parity import compare, compare_bwd, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
SPLIT = sm.SM_PLAN_SPLIT


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    sm.lib()


def _rand(M, N, dt, seed, scale=3.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(M, N, generator=g) * scale).to(TDT[dt])


def fwd(xd, out=None, **kw):
    if out is None:
        out = torch.full_like(xd, float("nan"))
    sm.softmax(xd, out=out, opts={"plan": SPLIT, **kw})
    torch.cuda.synchronize()
    return out


def bwd(yd, dyd, dx=None, **kw):
    if dx is None:
        dx = torch.full_like(yd, float("nan"))
    sm.softmax_backward(yd, dyd, dx=dx, opts={"plan": SPLIT, **kw})
    torch.cuda.synchronize()
    return dx


def test_wide_row_workload_full_size_auto():
    """64 x 131072 BF16 (per-row offsets U(-50, 50)): the automatic plan is SPLIT."""
    x = workloads.generate("offset_bf16_64x131072")
    xd = x.to(DEV)
    info = sm.plan_for(xd)
    assert info["plan_name"] == "split" and info["launches"] == 1
    before = sm.sync_failures()
    g = torch.full_like(xd, float("nan"))
    sm.softmax(xd, out=g)
    st = compare(g, x, what="offset_bf16_64x131072 split")
    log(f"[split] wide-row workload: plan {info}, {st}")
    assert sm.sync_failures() == before


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 4, 8])
def test_every_slice_shape(dt, V):
    for M, N in [(3, 1), (5, 7), (9, 1000), (4, 8193), (3, 20000), (2, 70001)]:
        x = _rand(M, N, dt, seed=N + V)
        for nt in (-1, 1):
            info = sm.plan_for(x.to(DEV), opts={"plan": SPLIT, "vecs_per_lane": V, "nontemporal": nt})
            assert info["vecs_per_lane"] == V and info["nt_loads"] == (nt == 1)
            g = fwd(x.to(DEV), vecs_per_lane=V, nontemporal=nt)
            compare(g, x, what=f"split {dt} V={V} nt={nt} {M}x{N} P={info['waves_per_row']}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rounds(dt):
    """A grid of one row's slices: every further row is another round."""
    M, N = 13, 20000
    x = _rand(M, N, dt, seed=5)
    xd = x.to(DEV)
    for V in (1, 2):
        P = sm.plan_for(xd, opts={"plan": SPLIT, "vecs_per_lane": V})["waves_per_row"]
        for grid in (P, 2 * P, 3 * P):
            info = sm.plan_for(xd, opts={"plan": SPLIT, "vecs_per_lane": V, "grid": grid})
            assert info["grid"] == grid
            g = fwd(xd, vecs_per_lane=V, grid=grid)
            compare(g, x, what=f"rounds {dt} V={V} grid={grid}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_masked_slices(dt):
    """Slices that are entirely -inf (shift 0, sum 0), a fully masked row, a row whose
    only live entry sits in the last slice, NaN and +inf confined to one slice."""
    M, N = 7, 9000
    x = _rand(M, N, dt, seed=8).float()
    x[0, :] = -math.inf
    x[1, : N - 1] = -math.inf
    x[2, 2048:6144] = -math.inf
    x[3, 4000] = math.nan
    x[4, 8999] = math.inf
    x[5, 1:] = -math.inf
    x = x.to(TDT[dt])
    for V in (1, 2):
        g = fwd(x.to(DEV), vecs_per_lane=V)
        compare(g, x, what=f"masked slices {dt} V={V}")
        gc = g.float().cpu()
        assert (gc[0] == 0).all() and gc[1, -1] == 1 and (gc[1, :-1] == 0).all()
        assert torch.isnan(gc[3]).all() and torch.isnan(gc[4]).all()
        assert gc[5, 0] == 1 and (gc[5, 1:] == 0).all()


def test_repeatable_and_misaligned():
    M, N = 11, 30001
    base = _rand(1, M * (N + 3) + 1, "bf16", seed=2).view(-1)
    x = base[1:1 + M * (N + 3)].view(M, N + 3)[:, :N]
    xd = base.to(DEV)[1:1 + M * (N + 3)].view(M, N + 3)[:, :N]
    ob = torch.full((M * (N + 5) + 2,), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = ob[2:2 + M * (N + 5)].view(M, N + 5)[:, :N]
    fwd(xd, out=out)
    compare(out, x.contiguous(), what="split misaligned phase-shifted")
    assert torch.isnan(ob[2:2 + M * (N + 5)].view(M, N + 5)[:, N:].float()).all()
    a = fwd(xd)
    b = fwd(xd)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_wait_budget_runs_out_out_of_place():
    """A wait budget of one poll (forced from the host): slices whose peers have not
    yet published give up, count the failure, and re-read their whole input row for
    the row statistics, so every element still matches the oracle. Every kernel drains."""
    M, N = 32, 131072
    x = _rand(M, N, "bf16", seed=3)
    xd = x.to(DEV)
    for dt in ("bf16", "f32"):
        xt = x.to(TDT[dt])
        xd = xt.to(DEV)
        before = sm.sync_failures()
        g = fwd(xd, vecs_per_lane=1, spin_limit=1)
        n = sm.sync_failures() - before
        compare(g, xt, what=f"{dt} one-poll budget, out of place")
        log(f"[split] {dt} one-poll budget out of place: {n} slices fell back to the whole row")
        assert n > 0
        # the default budget then works again on the same stream and slots
        after = sm.sync_failures()
        g = fwd(xd, vecs_per_lane=1)
        compare(g, xt, what=f"{dt} after timeouts")
        assert sm.sync_failures() == after


def test_wait_budget_runs_out_in_place():
    """In place, a slice that gives up cannot re-read its row (its peers may already
    have written theirs): each slice is then either correct or all NaN, and the
    failure count grows by the number of NaN slices."""
    M, N = 32, 131072
    x = _rand(M, N, "bf16", seed=4)
    xd = x.to(DEV)
    info = sm.plan_for(xd, opts={"plan": SPLIT, "vecs_per_lane": 1})
    P, S = info["waves_per_row"], 256 * 8
    before = sm.sync_failures()
    fwd(xd, out=xd, vecs_per_lane=1, spin_limit=1)
    after = sm.sync_failures()
    gc = xd.float().cpu().view(M, P, S)
    nan_slices = torch.isnan(gc).all(dim=2)
    partly = torch.isnan(gc).any(dim=2) & ~nan_slices
    assert not partly.any()
    assert after - before == int(nan_slices.sum())
    ok_rows = [i for i in range(M) if not nan_slices[i].any()]
    if ok_rows:
        compare(xd[ok_rows], x[ok_rows], what="in place: rows without timeouts")
    log(f"[split] one-poll budget in place: {int(nan_slices.sum())} of {M * P} slices timed out")


def test_backward_wait_budget_runs_out():
    """The backward with a one-poll budget: out of place, slices that give up form
    the row's dot product from y and dy themselves (oracle parity, failures counted);
    in place over dy, they write NaN and are counted."""
    M, N = 24, 131072
    y, dy = _bwd_inputs(M, N, "bf16", seed=8)
    yd, dyd = y.to(DEV), dy.to(DEV)
    before = sm.sync_failures()
    g = bwd(yd, dyd, vecs_per_lane=1, spin_limit=1)
    n = sm.sync_failures() - before
    compare_bwd(g, y, dy, what="bwd one-poll budget, out of place")
    log(f"[split] backward one-poll budget: {n} slices fell back to the whole row")
    assert n > 0
    before = sm.sync_failures()
    bwd(yd, dyd, dx=dyd, vecs_per_lane=1, spin_limit=1)
    n = sm.sync_failures() - before
    P = sm.plan_for_backward(yd, dyd, opts={"plan": SPLIT, "vecs_per_lane": 1})["waves_per_row"]
    gc = dyd.float().cpu().view(M, P, -1)
    nan_slices = torch.isnan(gc).all(dim=2)
    assert not (torch.isnan(gc).any(dim=2) & ~nan_slices).any()
    assert n == int(nan_slices.sum())


def test_two_streams_at_once():
    x1 = _rand(64, 65536, "bf16", seed=21)
    x2 = _rand(48, 40000, "f16", seed=22)
    d1, d2 = x1.to(DEV), x2.to(DEV)
    o1, o2 = torch.full_like(d1, float("nan")), torch.full_like(d2, float("nan"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(4):
        with torch.cuda.stream(s1):
            sm.softmax(d1, out=o1, opts={"plan": SPLIT})
        with torch.cuda.stream(s2):
            sm.softmax(d2, out=o2, opts={"plan": SPLIT})
    torch.cuda.synchronize()
    compare(o1, x1, what="stream 1")
    compare(o2, x2, what="stream 2")
    assert sm.sync_failures(s1) == 0 and sm.sync_failures(s2) == 0


# ------------------------------------------------------------------ backward

def _bwd_inputs(M, N, dt, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, N, generator=g, dtype=torch.float64) * 3
    y = torch.softmax(x, -1).to(TDT[dt])
    dy = torch.randn(M, N, generator=g, dtype=torch.float64).to(TDT[dt])
    return y, dy


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 4])
def test_backward_every_slice_shape(dt, V):
    for M, N in [(3, 1), (9, 1000), (4, 8193), (3, 20000), (2, 70001)]:
        y, dy = _bwd_inputs(M, N, dt, seed=N + V)
        for nt in (-1, 1):
            g = bwd(y.to(DEV), dy.to(DEV), vecs_per_lane=V, nontemporal=nt)
            compare_bwd(g, y, dy, what=f"bwd split {dt} V={V} nt={nt} {M}x{N}")


def test_backward_rounds_phase_and_in_place():
    M, N = 13, 20000
    y, dy = _bwd_inputs(M, N, "bf16", seed=4)
    yd, dyd = y.to(DEV), dy.to(DEV)
    P = sm.plan_for_backward(yd, dyd, opts={"plan": SPLIT, "vecs_per_lane": 1})["waves_per_row"]
    g = bwd(yd, dyd, vecs_per_lane=1, grid=P)
    compare_bwd(g, y, dy, what="bwd split rounds")
    # dy at another 16-byte phase (element loads), dx at another phase (element stores)
    db = torch.zeros(M * N + 3, dtype=torch.bfloat16, device=DEV)
    dv = db[3:].view(M, N)
    dv.copy_(dyd)
    xb = torch.full((M * N + 1,), float("nan"), dtype=torch.bfloat16, device=DEV)
    xv = xb[1:].view(M, N)
    bwd(yd, dv, dx=xv)
    compare_bwd(xv, y, dy, what="bwd split phases")
    bwd(yd, dyd, dx=dyd)
    compare_bwd(dyd, y, dy, what="bwd split in place over dy")


def test_backward_wide_row_shape_auto():
    y = sm.softmax(workloads.generate("offset_bf16_64x131072").to(DEV))
    dy = workloads.upstream_grad(y.shape, "bf16")
    info = sm.plan_for_backward(y, dy.to(DEV))
    assert info["plan_name"] == "split"
    before = sm.sync_failures()  # cumulative per stream
    dx = torch.full_like(y, float("nan"))
    sm.softmax_backward(y, dy.to(DEV), dx=dx)
    torch.cuda.synchronize()
    st = compare_bwd(dx, y.cpu(), dy, what="bwd 64x131072 split")
    log(f"[split] backward wide rows: {st}")
    assert sm.sync_failures() == before


def _each_plan(call, what):
    """Run ``call(plan)`` for the automatic plan, SPLIT and WIDE; a forced SPLIT may
    refuse rows whose slices cannot all be resident (SM_ERR_PLAN), nothing else.
    Returns the plans that ran."""
    ran = []
    for plan in (sm.SM_PLAN_AUTO, SPLIT, sm.SM_PLAN_WIDE):
        try:
            call(plan)
        except sm.SoftmaxError as e:
            assert plan == SPLIT and e.status == -7, (what, plan, e)
            continue
        ran.append(plan)
    assert sm.SM_PLAN_AUTO in ran and sm.SM_PLAN_WIDE in ran
    return ran


def _split_limit(query, lo, hi):
    """Largest row width N in [lo, hi) at which ``query(N)`` (a forced-SPLIT plan query
    for 2 BF16 rows, True when it succeeds) holds, by bisection; the query's success is
    monotone in N because every vector width needs more slices per row as N grows. The
    limit comes from the live occupancy of the SPLIT kernels on this device."""
    assert query(lo) and not query(hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if query(mid):
            lo = mid
        else:
            hi = mid
    return lo


def _fwd_split_fits(ptr):
    def q(N):
        rc, _ = sm.sm_softmax_plan_query(ptr, ptr, 2, N, N, N, sm.SM_BF16, {"plan": SPLIT})
        assert rc in (0, -7), rc
        return rc == 0
    return q


def _bwd_split_fits(ptr):
    def q(N):
        rc, _ = sm.sm_softmax_bwd_plan_query(ptr, ptr, ptr, 2, N, N, N, N, sm.SM_BF16,
                                             {"plan": SPLIT})
        assert rc in (0, -7), rc
        return rc == 0
    return q


def _widest_forward(N, split_expected):
    x = _rand(2, N, "bf16", seed=N % 997)
    xd = x.to(DEV)
    info = sm.plan_for(xd)
    log(f"[split] widest forward N={N}: auto plan {info['plan_name']} P={info['waves_per_row']}")
    before = sm.sync_failures()  # cumulative per stream

    def call(plan):
        out = torch.full_like(xd, float("nan"))
        sm.softmax(xd, out=out, opts={"plan": plan})
        torch.cuda.synchronize()
        compare(out, x, what=f"widest forward N={N} plan={plan}")
        del out

    ran = _each_plan(call, f"forward N={N}")
    assert (SPLIT in ran) == split_expected, (N, ran)
    assert info["plan_name"] == ("split" if split_expected else "wide")
    assert sm.sync_failures() == before


def _widest_backward(N, split_expected):
    y, dy = _bwd_inputs(2, N, "bf16", seed=N % 991)
    yd, dyd = y.to(DEV), dy.to(DEV)
    info = sm.plan_for_backward(yd, dyd)
    log(f"[split] widest backward N={N}: auto plan {info['plan_name']} P={info['waves_per_row']}")
    before = sm.sync_failures()  # cumulative per stream

    def call(plan):
        dx = torch.full_like(yd, float("nan"))
        sm.softmax_backward(yd, dyd, dx=dx, opts={"plan": plan})
        torch.cuda.synchronize()
        compare_bwd(dx, y, dy, what=f"widest backward N={N} plan={plan}")
        del dx

    ran = _each_plan(call, f"backward N={N}")
    assert (SPLIT in ran) == split_expected, (N, ran)
    assert info["plan_name"] == ("split" if split_expected else "wide")
    assert sm.sync_failures() == before


def test_widest_rows_forward():
    """The widest BF16 rows one launch of SPLIT can hold on this device (every slice of a
    row resident at once, from the SPLIT kernels' live occupancy) and one element past
    them, where the automatic plan falls back to the two-pass WIDE plan, plus a row of
    2^24 + 12345 elements: the automatic plan and both forced plans against the oracle."""
    buf = torch.empty(8, dtype=torch.bfloat16, device=DEV)
    lim = _split_limit(_fwd_split_fits(buf.data_ptr()), 1 << 16, 1 << 26)
    log(f"[split] forward SPLIT limit for 2 BF16 rows: N = {lim}")
    _widest_forward(lim, True)
    _widest_forward(lim + 1, False)
    _widest_forward((1 << 24) + 12345, False)


def test_widest_rows_backward():
    """As the forward test, for the backward's SPLIT limit (two inputs per element, so
    fewer vectors per lane)."""
    buf = torch.empty(8, dtype=torch.bfloat16, device=DEV)
    lim = _split_limit(_bwd_split_fits(buf.data_ptr()), 1 << 16, 1 << 26)
    log(f"[split] backward SPLIT limit for 2 BF16 rows: N = {lim}")
    _widest_backward(lim, True)
    _widest_backward(lim + 1, False)
    _widest_backward((1 << 23) + 7, False)


@pytest.mark.parametrize("M,N", [(4, 16385), (256, 32768), (64, 1 << 19)])
def test_fp32_automatic_plans(M, N):
    """The FP32 terms of the forward rule against the oracle: few rows split into slices
    of one vector per lane, 8192-window rows from 128 rows one-pass (1024 lanes x 8), and
    2^17-window rows over several SPLIT rounds on the two-pass plan (8 chunks per wave)."""
    x = _rand(M, N, "f32", seed=N % 991 + M)
    xd = x.to(DEV)
    info = sm.plan_for(xd)
    log(f"[split] fp32 {M}x{N}: plan {info['plan_name']} G={info['lanes_per_row']} "
        f"V={info['vecs_per_lane']} P={info['waves_per_row']} cpw={info['chunks_per_wave']}")
    if (M, N) == (4, 16385):
        assert (info["plan_name"], info["vecs_per_lane"]) == ("split", 1)
    if (M, N) == (256, 32768):
        assert (info["plan_name"], info["lanes_per_row"], info["vecs_per_lane"]) == ("persistent", 1024, 8)
    before = sm.sync_failures()  # cumulative per stream
    out = torch.full_like(xd, float("nan"))
    sm.softmax(xd, out=out)
    torch.cuda.synchronize()
    compare(out, x, what=f"fp32 auto {M}x{N} {info['plan_name']}")
    assert sm.sync_failures() == before
