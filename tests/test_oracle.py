"""Pins for the FP64 oracle, each against something other than the oracle itself.

The oracle computes the row softmax from its plain definition (subtract the row
maximum, exponentiate, divide by the sum: "Triton: Writing GPU Kernels in Python,
Measured", section "Step 2: a fused softmax") in FP64 and rounds once to the
storage dtype (Warpline README, the paragraph on the K2 reference). These tests
pin it with:

* independent decoders/encoders (numpy float16, torch bfloat16, numpy float32) and
  hand-built rounding ties, for the storage conversions;
* 50-digit ``decimal`` brute force on tiny rows;
* closed forms: constant rows, two-element rows (logistic), geometric rows,
  +/-1e4 spikes, the first causal row;
* invariants: row sums, shift invariance, strided views, row and column
  permutations, masked entries;
* a library special case: ``torch.softmax`` in float64 on the CPU.
"""
import decimal
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

DT = ["f32", "f16", "bf16"]
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def stored(x32, dtype):
    """float32/float64 values -> stored elements of ``dtype`` via torch (RNE)."""
    t = torch.as_tensor(np.asarray(x32, dtype=np.float32)).to(TORCH_DT[dtype])
    return workloads.storage_numpy(t)


# ------------------------------------------------------------------ conversions

def test_decode_f16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    # a few patterns by hand: 1.0, -2.0, smallest subnormal, +inf
    hand = oracle.decode(np.array([0x3F80, 0xC000, 0x0001, 0x7F80], np.uint16), "bf16")
    assert list(hand) == [1.0, -2.0, 2.0 ** -133, math.inf]


def test_decode_f32_patterns():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    got = oracle.decode(bits.view(np.float32), "f32")
    want = bits.view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def _probe_doubles(rng, n):
    """Doubles over many binades, plus exact halfway points and their neighbours."""
    mags = np.exp2(rng.uniform(-160, 140, size=n))
    vals = mags * rng.choice([-1.0, 1.0], size=n)
    return np.concatenate([vals, [0.0, -0.0, np.inf, -np.inf, 1e-320, -1e-320]])


def test_encode_f16_matches_numpy():
    rng = np.random.default_rng(2)
    v = _probe_doubles(rng, 200000)
    # halfway points between adjacent halves (including subnormal ones) and nudges
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = (h[:-1] + np.diff(h) / 2)
    v = np.concatenate([v, mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    got = oracle.encode(v, "f16")
    want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_f32_matches_numpy():
    rng = np.random.default_rng(3)
    v = _probe_doubles(rng, 200000)
    f = rng.standard_normal(5000).astype(np.float32).astype(np.float64)
    ulp = np.spacing(f.astype(np.float32)).astype(np.float64)
    v = np.concatenate([v, f + ulp / 2, f - ulp / 2, f + ulp / 2 * (1 + 2 ** -30),
                        [np.float64(np.float32(1e-45)) * 1.5]])
    got = oracle.encode(v, "f32")
    want = v.astype(np.float32).view(np.uint32)
    assert np.array_equal(got.view(np.uint32), want)


def test_encode_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    got = oracle.encode(f.astype(np.float64), "bf16")
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_rounds_once_from_double():
    one = 1.0
    cases = {
        one + 2 ** -8: 0x3F80,                # exact tie -> even (1.0)
        one + 3 * 2 ** -8: 0x3F82,            # exact tie -> even (1 + 2^-6)
        one + 2 ** -8 + 2 ** -40: 0x3F81,     # just above the tie: a float32 detour would give 1.0
        one + 2 ** -8 - 2 ** -40: 0x3F80,
        -(one + 2 ** -8 + 2 ** -40): 0xBF81,
        3.3895313892515355e38: 0x7F7F,        # largest finite bfloat16
        2.0 ** 128 - 2.0 ** 119: 0x7F80,      # max + half ulp: a tie, the even neighbour is inf
        2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100: 0x7F7F,
        2.0 ** -133: 0x0001,                  # smallest subnormal
        2.0 ** -134: 0x0000,                  # tie between 0 and the smallest subnormal -> 0
        2.0 ** -134 * (1 + 2 ** -20): 0x0001,
        2.0 ** -126 - 2.0 ** -140: 0x0080,    # rounds up into the smallest normal
    }
    got = oracle.encode(np.array(list(cases), np.float64), "bf16")
    assert [int(g) for g in got] == list(cases.values())
    nan = oracle.encode(np.array([np.nan]), "bf16")[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# ------------------------------------------------------------------ brute force

def _decimal_softmax(row):
    """50-digit softmax of a list of floats (exact decimal conversion of each)."""
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        finite = [decimal.Decimal(v) for v in row if v != -math.inf]
        if not finite:
            return [0.0] * len(row)
        m = max(finite)
        e = [decimal.Decimal(0) if v == -math.inf else (decimal.Decimal(v) - m).exp() for v in row]
        s = sum(e)
        return [float(v / s) for v in e]


@pytest.mark.parametrize("dtype", DT)
def test_brute_force_decimal_tiny_rows(dtype):
    rng = np.random.default_rng({"f32": 10, "f16": 11, "bf16": 12}[dtype])
    rows = []
    for k in range(300):
        n = int(rng.integers(1, 17))
        scale = [0.1, 1.0, 10.0, 100.0][k % 4]
        r = rng.standard_normal(n) * scale
        if k % 7 == 0 and n > 1:
            r[rng.integers(0, n)] = -np.inf
        if k % 11 == 0:
            r[:] = r[0]  # all equal
        if k % 13 == 0 and n > 2:
            r[1] = r[2]  # duplicates
        if dtype == "f16":
            r = np.clip(r, -60000, 60000)
        rows.append(r)
    for r in rows:
        s = stored(r[None, :], dtype)
        y = oracle.softmax_f64(s, dtype)[0]
        x = oracle.decode(s, dtype)[0]
        want = np.array(_decimal_softmax([float(v) for v in x]))
        assert np.all(np.abs(y - want) <= 1e-12 * np.abs(want) + 1e-300), (dtype, x, y, want)


# ------------------------------------------------------------------ closed forms

@pytest.mark.parametrize("dtype", DT)
@pytest.mark.parametrize("n", [1, 7, 781, 4096])
@pytest.mark.parametrize("c", [0.0, 1.5, -3.0, 1e4])
def test_constant_row_is_one_over_n(dtype, n, c):
    s = stored(np.full((3, n), c), dtype)
    y, yr = oracle.reference(s, dtype)
    assert np.all(y == 1.0 / n)
    want = {"f32": np.float32(1.0 / n).view(np.uint32),
            "f16": np.float16(1.0 / n).view(np.uint16)}.get(dtype)
    if want is not None:
        assert np.all(yr.view(want.dtype) == want)


def test_two_element_rows_are_logistic():
    rng = np.random.default_rng(5)
    ab = rng.uniform(-30, 30, size=(500, 2)).astype(np.float32)
    y = oracle.softmax_f64(ab, "f32")
    a = ab[:, 0].astype(np.float64)
    b = ab[:, 1].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(b - a))
    assert np.allclose(y[:, 0], sig, rtol=1e-14, atol=0)
    assert np.allclose(y[:, 1], 1.0 / (1.0 + np.exp(a - b)), rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype,n", [("bf16", 256), ("f16", 1024), ("f32", 4096)])
def test_geometric_row_closed_form(dtype, n):
    d = 1.0 / 8.0
    j = np.arange(n, dtype=np.float64)
    s = stored((j * d)[None, :], dtype)
    assert np.array_equal(oracle.decode(s, dtype)[0], j * d)  # the grid is exact
    y = oracle.softmax_f64(s, dtype)[0]
    # y_j = r^j (r - 1) / (r^n - 1) with r = e^d, written as
    # e^{(j-n+1)d} (1 - e^{-d}) / (1 - e^{-nd}) so that nothing overflows
    want = np.exp((j - n + 1) * d) * (-np.expm1(-d)) / (-np.expm1(-n * d))
    assert np.allclose(y, want, rtol=1e-12, atol=1e-300)


def test_spikes_give_exact_fractions():
    rng = np.random.default_rng(6)
    for k in [1, 2, 3, 5]:
        x = rng.uniform(-8, 8, size=(4, 1000)).astype(np.float32)
        pos = rng.choice(1000, size=k, replace=False)
        x[:, pos] = 1e4
        neg = rng.choice(np.setdiff1d(np.arange(1000), pos), size=4, replace=False)
        x[:, neg] = -1e4
        s = stored(x, "f16")
        y = oracle.softmax_f64(s, "f16")
        assert np.all(y[:, pos] == 1.0 / k)
        rest = np.setdiff1d(np.arange(1000), pos)
        assert np.all(y[:, rest] == 0.0)
    # only negative spikes: they give exactly 0 and the rest is an ordinary softmax
    x = rng.uniform(-8, 8, size=(2, 300)).astype(np.float32)
    x[:, :10] = -1e4
    s = stored(x, "f16")
    y = oracle.softmax_f64(s, "f16")
    assert np.all(y[:, :10] == 0.0)
    sub = oracle.softmax_f64(s[:, 10:], "f16")
    assert np.allclose(y[:, 10:], sub, rtol=1e-15, atol=0)


def test_causal_first_rows():
    head = workloads.causal_head(0, 0, shape=(1, 1, 64, 64, 128))
    s = workloads.storage_numpy(head)
    y = oracle.softmax_f64(s, "bf16")
    assert np.array_equal(y[0], np.eye(64)[0])
    x = oracle.decode(s, "bf16")
    d = x[1, 0] - x[1, 1]
    assert math.isclose(y[1, 0], 1.0 / (1.0 + math.exp(-d)), rel_tol=1e-14)
    assert math.isclose(y[1, 1], 1.0 / (1.0 + math.exp(d)), rel_tol=1e-14)
    assert np.all(np.triu(y, 1) == 0.0)


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("dtype", DT)
def test_row_sums_and_range(dtype):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 3000)) * 5
    y = oracle.softmax_f64(stored(x, dtype), dtype)
    assert np.all((y >= 0) & (y <= 1))
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) <= 3000 * 2 ** -52


def test_shift_invariance_is_bitwise():
    rng = np.random.default_rng(8)
    x = rng.integers(-8, 9, size=(16, 500)).astype(np.float32)
    a = oracle.softmax_f64(stored(x, "bf16"), "bf16")
    b = oracle.softmax_f64(stored(x + 64, "bf16"), "bf16")
    assert np.array_equal(a, b)
    xf = (rng.integers(-512, 513, size=(16, 500)) / 64).astype(np.float32)
    assert np.array_equal(oracle.softmax_f64(xf, "f32"), oracle.softmax_f64(xf - 3.25, "f32"))


def test_rows_are_independent_and_indexed_right():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 333)) + rng.uniform(-20, 20, size=(40, 1))).astype(np.float32)
    full = oracle.softmax_f64(x, "f32")
    for i in [0, 1, 17, 39]:
        assert np.array_equal(full[i], oracle.softmax_f64(x[i:i + 1], "f32")[0])
    perm = rng.permutation(40)
    assert np.array_equal(oracle.softmax_f64(x[perm], "f32"), full[perm])
    picked = oracle.softmax_f64(x, "f32", rows=[39, 0, 5, 5])
    assert np.array_equal(picked, full[[39, 0, 5, 5]])
    # reversing the columns reverses the output (the sum order changes: tolerance)
    rev = oracle.softmax_f64(np.ascontiguousarray(x[:, ::-1]), "f32")
    assert np.allclose(rev[:, ::-1], full, rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", DT)
def test_strided_view_matches_contiguous(dtype):
    rng = np.random.default_rng(10)
    big = stored(rng.standard_normal((30, 517)) * 3, dtype)
    view = big[:, 5:5 + 400]
    assert view.strides[0] == 517 * view.itemsize
    assert np.array_equal(oracle.softmax_f64(view, dtype),
                          oracle.softmax_f64(np.ascontiguousarray(view), dtype))


def test_masked_entries_and_special_rows():
    x = np.array([
        [0.0, -np.inf, 1.0, -np.inf],     # masked entries -> exactly 0
        [-np.inf] * 4,                    # fully masked row -> zeros (reading)
        [np.nan, 0.0, 1.0, 2.0],          # NaN -> whole row NaN
        [np.inf, 0.0, 1.0, 2.0],          # +inf -> whole row NaN
        [np.nan, -np.inf, -np.inf, -np.inf],
    ], np.float32)
    y = oracle.softmax_f64(x, "f32")
    assert y[0, 1] == 0.0 and y[0, 3] == 0.0
    assert math.isclose(y[0, 2], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert np.all(y[1] == 0.0)
    assert np.all(np.isnan(y[2])) and np.all(np.isnan(y[3])) and np.all(np.isnan(y[4]))


def test_monotone_within_row():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 1000)).astype(np.float32)
    y = oracle.softmax_f64(x, "f32")
    for i in range(8):
        o = np.argsort(x[i], kind="stable")
        assert np.all(np.diff(y[i][o]) >= 0)


def test_empty_shapes():
    assert oracle.softmax_f64(np.zeros((0, 5), np.float32), "f32").shape == (0, 5)
    assert oracle.softmax_f64(np.zeros((3, 0), np.float32), "f32").shape == (3, 0)


@pytest.mark.parametrize("dtype", DT)
def test_agrees_with_torch_float64_softmax(dtype):
    rng = np.random.default_rng(12)
    s = stored(rng.standard_normal((64, 1000)) * 4, dtype)
    y = oracle.softmax_f64(s, dtype)
    xt = torch.from_numpy(oracle.decode(s, dtype))
    want = torch.softmax(xt, dim=-1).numpy()
    assert np.allclose(y, want, rtol=1e-13, atol=1e-300)


def test_threads_do_not_change_results():
    x = workloads.storage_numpy(workloads.spiky_f16(256, M=512))
    a = oracle.softmax_f64(x, "f16", threads=1)
    b = oracle.softmax_f64(x, "f16", threads=4)
    assert np.array_equal(a, b)
