"""The forward comparison's gates, on the CPU: the README tolerance (atol = rtol =
4e-3 for FP16/BF16) and the tighter one-ulp gate against the oracle's rounded
result. A correct output passes, a neighbour on the dtype grid passes, and an
output two units in the last place away fails, on probabilities small enough that
the 4e-3 absolute term alone would have let it through."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare, rel_thr_bound, ulp

TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def test_ulp_of_the_grid():
    # BF16: 7 fraction bits, normal range from 2^-126, subnormal spacing 2^-133
    r = np.array([1.0, 0.75, 0.5, 2.0 ** -126, 2.0 ** -130, 0.0, 3.0e38])
    want = np.array([2.0 ** -7, 2.0 ** -8, 2.0 ** -8, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133,
                     2.0 ** (127 - 7)])
    assert np.array_equal(ulp(r, "bf16"), want)
    # FP16: 10 fraction bits, normal range from 2^-14, subnormal spacing 2^-24
    r = np.array([1.0, 0.999, 2.0 ** -14, 6.0e-5, 2.0 ** -24, 0.0, 65504.0])
    want = np.array([2.0 ** -10, 2.0 ** -11, 2.0 ** -24, 2.0 ** -25 * 2, 2.0 ** -24, 2.0 ** -24,
                     32.0])
    assert np.array_equal(ulp(r, "f16"), want)
    # every step between neighbours of the grid is one ulp of the lower one
    for dt, bits in (("bf16", np.arange(1, 0x7F7F, 97, dtype=np.uint16)),
                     ("f16", np.arange(1, 0x7BFF, 89, dtype=np.uint16))):
        lo = oracle.decode(bits, dt)
        hi = oracle.decode(bits + 1, dt)
        assert np.array_equal(hi - lo, ulp(lo, dt)), dt


def _correct_output(dt):
    x = workloads.normal_bf16_4096x4096(M=64, N=4096).float().to(TDT[dt])
    _, yr = oracle.reference(workloads.storage_numpy(x), dt)
    g = torch.from_numpy(yr.view(np.int16)).view(TDT[dt])
    return x, g, yr


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_rounded_oracle_and_its_neighbour_pass(dt):
    x, g, yr = _correct_output(dt)
    st = compare(g, x, what="rounded oracle")
    assert st["max_ulp_vs_rounded"] == 0.0
    assert st["max_rel_thr"] <= rel_thr_bound(dt)
    # one step up on a small probability: within the gate
    i, j = np.unravel_index(np.argmin(np.abs(oracle.decode(yr, dt) - 3e-4)), yr.shape)
    bits = yr.copy()
    bits[i, j] += 1
    st = compare(torch.from_numpy(bits.view(np.int16)).view(TDT[dt]), x, what="one ulp")
    assert st["max_ulp_vs_rounded"] == 1.0


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("target", [3e-4, 0.02])
def test_two_ulps_off_fails(dt, target):
    x, _, yr = _correct_output(dt)
    ref = oracle.decode(yr, dt)
    i, j = np.unravel_index(np.argmin(np.abs(ref - target)), yr.shape)
    bits = yr.copy()
    bits[i, j] += 2  # two steps up within the binade (positive values)
    moved = oracle.decode(bits[i, j:j + 1], dt)[0]
    assert moved - ref[i, j] == 2 * ulp(ref[i:i + 1, j], dt)[0]
    if target < 1e-3:  # the README tolerance alone would not see it
        assert moved - ref[i, j] <= 4e-3 + 4e-3 * ref[i, j]
    with pytest.raises(AssertionError, match="more than one ulp"):
        compare(torch.from_numpy(bits.view(np.int16)).view(TDT[dt]), x, what="two ulps")


def test_bf16_floor_below_the_fp32_normal_range():
    """A BF16 result the FP32 exponential flushes to 0 (exact value below 2^-126) is
    within the gate's floor; the same error on a normal value is not."""
    x = torch.tensor([[0.0, -86.0, -90.0, -3.0]]).to(torch.bfloat16)
    _, yr = oracle.reference(workloads.storage_numpy(x), "bf16")
    ref = oracle.decode(yr, "bf16")
    assert 0 < ref[0, 2] < 2.0 ** -126 < ref[0, 1]
    bits = yr.copy()
    bits[0, 2] = 0  # flushed
    compare(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16), x, what="flushed")
    bits = yr.copy()
    bits[0, 1] = 0
    with pytest.raises(AssertionError):
        compare(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16), x, what="zeroed")
