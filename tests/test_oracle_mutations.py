"""Planted mistakes: each one, compiled into a scratch copy of the oracle on the CPU,
must fail at least one pin. This shows that the pins constrain every step of the
oracle (decode, max, exp, sum, divide, row indexing, the all--inf reading, the
one-step RNE encode, the backward, the residual RMSNorm, the attention), not just its
happy path.

The mutants are built from the committed C source with plain text edits and gcc;
nothing here touches the GPU or the GPU library.
"""
import decimal
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle

SRC = os.path.join(os.path.dirname(oracle.LIB_PATH), "oracle_softmax.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("no max shift", "y[j] = exp(x[j] - m);", "y[j] = exp(x[j]);"),
    ("wrong sign in exponent", "y[j] = exp(x[j] - m);", "y[j] = exp(m - x[j]);"),
    ("max skips first entry", "for (int64_t j = 0; j < n; ++j)\n        if (x[j] > m)",
     "for (int64_t j = 1; j < n; ++j)\n        if (x[j] > m)"),
    ("sum drops a term", "        s += y[j];\n", "        if (j + 1 < n) s += y[j];\n"),
    ("sum in float", "    double s = 0.0;", "    float s = 0.0f;"),
    ("divides by n", "y[j] = y[j] / s;", "y[j] = y[j] / (double)n;"),
    ("row index ignores stride", "base + (size_t)(r * in_stride)", "base + (size_t)(r * cols)"),
    ("f16 exponent bias", "ex - 25", "ex - 24"),
    ("f16 subnormal scale", "ldexp((double)fr, -24)", "ldexp((double)fr, -25)"),
    ("bf16 decode shift", "(uint32_t)b << 16", "(uint32_t)b << 15"),
    ("encode truncates", "double r = nearbyint(", "double r = trunc("),
    ("encode ties away", "double r = nearbyint(", "double r = round("),
    ("encode drops carry", "        r = ldexp(1.0, mant);\n        E += 1;", "        r = ldexp(1.0, mant + 1) - 1;"),
    ("all -inf row gives NaN", "y[j] = has_nan ? NAN : 0.0;", "y[j] = NAN;"),
    ("NaN ignored", "y[j] = has_nan ? NAN : 0.0;", "y[j] = 0.0;"),
    ("bwd wrong sign", "dx[j] = y[j] * (dy[j] - d);", "dx[j] = y[j] * (d - dy[j]);"),
    ("bwd drops a dot term", "for (int64_t j = 0; j < n; ++j) d += y[j] * dy[j];",
     "for (int64_t j = 1; j < n; ++j) d += y[j] * dy[j];"),
    ("bwd scales by dy", "dx[j] = y[j] * (dy[j] - d);", "dx[j] = dy[j] * (dy[j] - d);"),
    ("bwd dy stride", "db + (size_t)(r * dy_stride)", "db + (size_t)(r * y_stride)"),
    ("rms ignores residual", "encode_binary(v + load_elem(rr + (size_t)j * es, dtype),",
     "encode_binary(v,"),
    ("rms sum not rounded", "v = load_elem(buf, dtype);",
     "v = v + load_elem(rr + (size_t)j * es, dtype);"),
    ("rms drops eps", "sqrt(q / (double)n + eps)", "sqrt(q / (double)n)"),
    ("rms mean over n - 1", "sqrt(q / (double)n + eps)", "sqrt(q / (double)(n - 1) + eps)"),
    ("rms ignores weight", "y[j] = sv[j] * w[j] / den;", "y[j] = sv[j] / den;"),
    ("rms no square root", "sqrt(q / (double)n + eps)", "(q / (double)n + eps)"),
    ("rms weight index", "a[cols + j] = load_elem(wb + (size_t)j * es, dtype);",
     "a[cols + j] = load_elem(wb, dtype);"),
    ("rms residual stride", "(size_t)(row * r_stride)", "(size_t)(row * x_stride)"),
    ("attn drops scale", "sv[j] = scale * acc;", "sv[j] = acc;"),
    ("attn mask off by one", "if (causal && j > i + (Sk - Sq))", "if (causal && j >= i + (Sk - Sq))"),
    ("attn mask top-left", "if (causal && j > i + (Sk - Sq))", "if (causal && j > i)"),
    ("attn reads k for v", "vb + (size_t)(h * v_hs + j * v_rs + c)", "kb + (size_t)(h * k_hs + j * k_rs + c)"),
    ("attn k head stride", "kb + (size_t)(h * k_hs", "kb + (size_t)(h * q_hs"),
    ("attn lse drops max", "lse[t] = m + log(ssum);", "lse[t] = log(ssum);"),
]


def _stored(x, dtype):
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(tdt)
    return t.numpy() if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


def _decimal_softmax(row):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        fin = [decimal.Decimal(v) for v in row if v != -math.inf]
        m = max(fin)
        e = [decimal.Decimal(0) if v == -math.inf else (decimal.Decimal(v) - m).exp() for v in row]
        s = sum(e)
        return np.array([float(v / s) for v in e])


def pin_battery(orc: "oracle.Oracle"):
    """A compact subset of the oracle pins; returns the names of those that fail."""
    failed = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    rng = np.random.default_rng(99)

    def brute():
        for dtype in ("f32", "f16", "bf16"):
            for _ in range(40):
                n = int(rng.integers(2, 12))
                s = _stored(rng.standard_normal((1, n)) * 4, dtype)
                x = orc.decode(s, dtype)[0]
                y = orc.softmax_f64(s, dtype)[0]
                want = _decimal_softmax(list(x))
                if not np.all(np.abs(y - want) <= 1e-12 * want + 1e-300):
                    return False
        return True

    def f16_decode():
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        got, want = orc.decode(bits, "f16"), bits.view(np.float16).astype(np.float64)
        ok = ~np.isnan(want)
        return np.array_equal(got[ok], want[ok])

    def bf16_decode():
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
        got = orc.decode(bits, "bf16")
        ok = ~np.isnan(want)
        return np.array_equal(got[ok], want[ok])

    def encode_f16():
        v = np.exp2(rng.uniform(-30, 17, 20000)) * rng.choice([-1.0, 1.0], 20000)
        h = np.arange(0, 0x7C00, 3, dtype=np.uint16).view(np.float16).astype(np.float64)
        v = np.concatenate([v, h[:-1] + np.diff(h) / 2])
        return np.array_equal(orc.encode(v, "f16"), v.astype(np.float16).view(np.uint16))

    def constant_rows():
        for c in (0.0, 1e4):
            y = orc.softmax_f64(_stored(np.full((2, 781), c), "f32"), "f32")
            if not np.all(y == 1.0 / 781):
                return False
        return True

    def spikes_first_last():
        x = rng.uniform(-8, 8, size=(2, 64)).astype(np.float32)
        x[0, 0] = 1e4
        x[1, -1] = 1e4
        y = orc.softmax_f64(_stored(x, "f16"), "f16")
        return y[0, 0] == 1.0 and y[1, -1] == 1.0 and np.sum(y) == 2.0

    def strided():
        big = _stored(rng.standard_normal((9, 40)), "bf16")
        v = big[:, 3:33]
        return np.array_equal(orc.softmax_f64(v, "bf16"),
                              orc.softmax_f64(np.ascontiguousarray(v), "bf16"))

    def row_sums():
        y = orc.softmax_f64(_stored(rng.standard_normal((8, 3000)) * 5, "f32"), "f32")
        return np.max(np.abs(y.sum(1) - 1)) <= 3000 * 2 ** -52

    def masked():
        x = np.array([[-np.inf] * 4, [np.nan, 0, 1, 2], [np.nan] + [-np.inf] * 3], np.float32)
        y = orc.softmax_f64(x, "f32")
        return np.all(y[0] == 0.0) and np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))

    def bwd_torch():
        x = rng.standard_normal((4, 40)) * 2
        ys = _stored(torch.softmax(torch.from_numpy(x), -1).numpy(), "f32")
        g = _stored(rng.standard_normal((4, 40)), "f32")
        dx = orc.softmax_bwd_f64(ys, g, "f32")
        want = torch._softmax_backward_data(torch.from_numpy(g.astype(np.float64)),
                                            torch.from_numpy(ys.astype(np.float64)), -1,
                                            torch.float64).numpy()
        return np.allclose(dx, want, rtol=1e-12, atol=1e-15)

    def bwd_strided():
        yb = _stored(rng.random((6, 50)), "f32")
        gb = _stored(rng.standard_normal((6, 60)), "f32")
        return np.array_equal(orc.softmax_bwd_f64(yb[:, :40], gb[:, 5:45], "f32"),
                              orc.softmax_bwd_f64(np.ascontiguousarray(yb[:, :40]),
                                                  np.ascontiguousarray(gb[:, 5:45]), "f32"))

    def rms_torch():
        import torch.nn.functional as F
        for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            g = torch.Generator().manual_seed(5)
            x = (torch.randn(4, 33, generator=g) * 3).to(tdt)
            r = (torch.randn(4, 33, generator=g) * torch.exp2(torch.randint(-10, 2, (4, 33), generator=g))).to(tdt)
            w = torch.randn(33, generator=g).to(tdt)
            st = lambda t: t.numpy() if dt == "f32" else t.view(torch.int16).numpy().view(np.uint16)
            y, _ = orc.rmsnorm_f64(st(x), st(r), st(w), dt, 1e-2)
            want = F.rms_norm((x.float() + r.float()).to(tdt).double(), (33,), weight=w.double(),
                              eps=1e-2).numpy()
            if not np.allclose(y, want, rtol=1e-13, atol=0):
                return False
        return True

    def rms_strided():
        g = torch.Generator().manual_seed(6)
        xb, rb = torch.randn(5, 40, generator=g), torch.randn(5, 60, generator=g)
        w = torch.randn(30, generator=g)
        a, _ = orc.rmsnorm_f64(xb.numpy()[:, :30], rb.numpy()[:, 7:37], w.numpy(), "f32", 1e-6)
        b, _ = orc.rmsnorm_f64(np.ascontiguousarray(xb.numpy()[:, :30]),
                               np.ascontiguousarray(rb.numpy()[:, 7:37]), w.numpy(), "f32", 1e-6)
        return np.array_equal(a, b)

    def attn_torch():
        import torch.nn.functional as F
        g = torch.Generator().manual_seed(8)
        q = torch.randn(2, 6, 8, generator=g).to(torch.bfloat16)
        k = torch.randn(2, 9, 8, generator=g).to(torch.bfloat16)
        v = torch.randn(2, 9, 8, generator=g).to(torch.bfloat16)
        stn = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
        o, lse = orc.attention_f64(stn(q), stn(k), stn(v), "bf16", 0.3, True)
        mask = torch.arange(9)[None, :] <= torch.arange(6)[:, None] + 3
        want = F.scaled_dot_product_attention(q.double(), k.double(), v.double(), attn_mask=mask,
                                              scale=0.3).reshape(12, 8).numpy()
        s = (torch.einsum("hid,hjd->hij", q.double(), k.double()) * 0.3).masked_fill(~mask, -math.inf)
        wl = torch.logsumexp(s, -1).reshape(12).numpy()
        return np.allclose(o, want, rtol=1e-12, atol=1e-14) and np.allclose(lse, wl, rtol=1e-13)

    for name, fn in [("attn vs torch", attn_torch), ("rms vs torch", rms_torch), ("rms strided", rms_strided),
                     ("bwd vs torch", bwd_torch), ("bwd strided", bwd_strided),
                     ("brute force", brute), ("f16 decode", f16_decode), ("bf16 decode", bf16_decode),
                     ("f16 encode", encode_f16), ("constant rows", constant_rows),
                     ("spikes at the ends", spikes_first_last), ("strided view", strided),
                     ("row sums", row_sums), ("masked rows", masked)]:
        check(name, fn)
    return failed


def _build(tmp_path, text, tag):
    src = tmp_path / f"mut_{tag}.c"
    lib = tmp_path / f"libmut_{tag}.so"
    src.write_text(text)
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    str(src), "-o", str(lib), "-lm"], check=True, capture_output=True)
    return oracle.Oracle(str(lib))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_unmodified_oracle_passes_the_battery():
    assert pin_battery(oracle.default()) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name!r} not unique in the oracle source"
    orc = _build(tmp_path, text.replace(old, new), abs(hash(name)) % 10 ** 8)
    failed = pin_battery(orc)
    assert failed, f"planted mistake {name!r} passed every pin"
