"""The allocation-free forward (sm_softmax_fwd_noalloc) through the C ABI against
sm_softmax_fwd on the same inputs, and against the FP64 oracle: each case runs two
calls in a row on one device, the second on a smaller input, so the second reuses
the scratch array the first left behind (SPLIT slots and WIDE partial statistics)."""
import pytest
import torch

import memory_bound_row_sm_amd as sm
from parity import compare, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CODE = {"f32": sm.SM_F32, "f16": sm.SM_F16, "bf16": sm.SM_BF16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    sm.lib()


def _rand(M, N, dt, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, N, generator=g) * 3
    x += torch.empty(M, 1).uniform_(-50, 50, generator=g)  # per-row offsets
    return x.to(TDT[dt])


def _call(fn, x, out, dt):
    s = torch.cuda.current_stream().cuda_stream
    M, N = x.shape
    return fn(x.data_ptr(), out.data_ptr(), M, N, x.stride(0), out.stride(0), CODE[dt], s)


# (first shape, second smaller shape, dtype): SPLIT rows, WIDE rows (FP32 past the
# SPLIT capacity), and one-pass rows (no scratch)
CASES = [((64, 131072), (16, 40000), "bf16"),
         ((8, 1 << 20), (3, 100000), "f16"),
         ((256, 1 << 20), (4, 300000), "f32"),
         ((4096, 4096), (128, 781), "bf16")]


@pytest.mark.parametrize("first,second,dt", CASES)
def test_two_calls_match_sm_softmax_fwd(first, second, dt):
    for k, (M, N) in enumerate((first, second)):
        x = _rand(M, N, dt, seed=M + N + k)
        xd = x.to(DEV)
        plan = sm.plan_for(xd)["plan_name"]
        want = torch.full_like(xd, float("nan"))
        assert _call(sm.sm_softmax_fwd, xd, want, dt) == 0
        got = torch.full_like(xd, float("nan"))
        rc = _call(sm.sm_softmax_fwd_noalloc, xd, got, dt)
        torch.cuda.synchronize()
        assert rc == 0, sm.sm_softmax_strerror(rc)
        st = compare(got, x, what=f"noalloc {dt} {M}x{N} call {k}")
        compare(want, x, what=f"sm_softmax_fwd {dt} {M}x{N}")
        # same plan, same kernels: the same bits (a SPLIT fallback would change the
        # summation order, so allow the oracle bar there)
        same = torch.equal(got.view(torch.int8 if dt == "f32" else torch.int16),
                           want.view(torch.int8 if dt == "f32" else torch.int16))
        log(f"[noalloc] {dt} {M}x{N} call {k}: plan {plan}, identical bits {same}, {st}")


def test_in_place_takes_the_two_pass_plan():
    """In place, rows AUTO would split run on WIDE: two calls in a row, the second
    smaller, each against the oracle and against sm_softmax_fwd in place."""
    for k, (M, N) in enumerate(((32, 131072), (5, 50000))):
        x = _rand(M, N, "bf16", seed=7 + k)
        a, b = x.to(DEV), x.to(DEV)
        assert _call(sm.sm_softmax_fwd_noalloc, a, a, "bf16") == 0
        assert _call(sm.sm_softmax_fwd, b, b, "bf16") == 0
        torch.cuda.synchronize()
        compare(a, x, what=f"noalloc in place {M}x{N}")
        compare(b, x, what=f"sm_softmax_fwd in place {M}x{N}")


def test_scratch_limit_is_refused():
    """A plan whose workspace exceeds the array returns SM_ERR_WORKSPACE before
    launching anything: the output keeps its NaN fill."""
    M, N = 1024, 1 << 20
    x = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    need = sm.plan_for(x, out)["workspace_bytes"]
    assert need > sm.NOALLOC_SCRATCH_BYTES
    assert _call(sm.sm_softmax_fwd_noalloc, x, out, "bf16") == -6
    torch.cuda.synchronize()
    assert torch.isnan(out[:: 97, :: 4099].float()).all()
    del x, out
    torch.cuda.empty_cache()


def test_captured_and_replayed():
    """Captured into a graph (the call allocates nothing; rows AUTO would split run on
    WIDE under capture) and replayed on new inputs, with eager calls between."""
    M, N = 16, 65536
    xs = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    ys = torch.empty_like(xs)
    xs.copy_(_rand(M, N, "bf16", seed=1).to(DEV))
    assert _call(sm.sm_softmax_fwd_noalloc, xs, ys, "bf16") == 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert _call(sm.sm_softmax_fwd_noalloc, xs, ys, "bf16") == 0
    for i in range(3):
        x = _rand(M, N, "bf16", seed=50 + i)
        xs.copy_(x.to(DEV))
        ys.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare(ys, x, what=f"noalloc replay {i}")
        e = torch.full_like(xs, float("nan"))
        assert _call(sm.sm_softmax_fwd_noalloc, xs, e, "bf16") == 0  # eager, SPLIT
        torch.cuda.synchronize()
        compare(e, x, what=f"noalloc eager after replay {i}")
