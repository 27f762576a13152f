"""Seeded synthetic inputs for the row-softmax workloads.

This module holds no softmax arithmetic. It only draws random numbers, builds the
attention-shaped logits (q . k^T / sqrt(d) with a causal -inf mask) and casts to
the storage dtype with torch's round-to-nearest-even. The tests, the smoke check
and the bench take their inputs from here, and both the GPU library and the FP64
oracle consume the very same stored tensors.

Every generator is a pure function of its seed (numpy PCG64 through
``numpy.random.default_rng``), so a workload is identified by its recipe and the
SHA-256 of its stored bytes.

Workloads (the shapes, dtypes and value distributions of the method's headline
cases):

* ``normal_f32_128x781``      FP32 128 x 781, x ~ N(0, 1), seed 0 (a width that is
                              not a power of two and whose rows are not 16-byte aligned)
* ``normal_bf16_4096x4096``   BF16 4096 x 4096, x ~ N(0, 2^2), seed 2026
* ``spiky_f16_8192xN``        FP16 8192 x N for N in {127, 256, 1000, 2048, 4096, 8192},
                              x ~ U(-8, 8); each entry independently (p = 0.01) replaced
                              by +1e4 or -1e4 (sign p = 1/2); seed 2026, reset per N
* ``offset_bf16_64x131072``   BF16 64 x 131072, x ~ N(0, 1) plus a per-row offset
                              ~ U(-50, 50); seed 2026
* ``causal_bf16_524288x2048`` BF16 8 batches x 32 heads x 2048 queries x 2048 keys,
                              flattened to 524288 x 2048 rows; per head q and k ~ N(0, 1)
                              of shape 2048 x 128 (q drawn first), x = q k^T / sqrt(128)
                              in FP32, entries with key > query set to -inf; seed 2026
                              combined with (batch, head)
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np
import torch

SPIKE_WIDTHS = (127, 256, 1000, 2048, 4096, 8192)
CAUSAL_SHAPE = (8, 32, 2048, 2048, 128)  # batch, heads, queries, keys, head dim

_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    M: int
    N: int
    recipe: str


def _cast(x32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t if dtype == "f32" else t.to(_TORCH[dtype])


def normal_f32_128x781(M: int = 128, N: int = 781, seed: int = 0) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return _cast(rng.standard_normal((M, N), dtype=np.float32), "f32")


def normal_bf16_4096x4096(M: int = 4096, N: int = 4096, seed: int = 2026) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return _cast(2.0 * rng.standard_normal((M, N), dtype=np.float32), "bf16")


def spiky_f16(N: int, M: int = 8192, seed: int = 2026, dtype: str = "f16") -> torch.Tensor:
    rng = np.random.default_rng(seed)
    x = rng.uniform(-8.0, 8.0, size=(M, N)).astype(np.float32)
    spike = rng.random((M, N)) < 0.01
    sign = rng.random((M, N)) < 0.5
    x[spike] = np.where(sign[spike], np.float32(1e4), np.float32(-1e4))
    return _cast(x, dtype)


def offset_bf16_64x131072(M: int = 64, N: int = 131072, seed: int = 2026) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, N), dtype=np.float32)
    off = rng.uniform(-50.0, 50.0, size=(M, 1)).astype(np.float32)
    return _cast(x + off, "bf16")


def causal_head(b: int, h: int, seed: int = 2026, shape=CAUSAL_SHAPE) -> torch.Tensor:
    """The (queries x keys) BF16 logits of one (batch, head)."""
    _, _, nq, nk, d = shape
    rng = np.random.default_rng([seed, b, h])
    q = torch.from_numpy(rng.standard_normal((nq, d), dtype=np.float32))
    k = torch.from_numpy(rng.standard_normal((nk, d), dtype=np.float32))
    x = (q @ k.T) / math.sqrt(d)
    mask = torch.ones(nq, nk, dtype=torch.bool).triu(1)  # key index > query index
    x.masked_fill_(mask, float("-inf"))
    return x.to(torch.bfloat16)


def causal_bf16(seed: int = 2026, shape=CAUSAL_SHAPE, heads=None) -> torch.Tensor:
    """Flattened causal logits, rows ordered ((b * H + h) * Q + i).

    ``heads``: optional list of flat head indices (b * H + h) to build; the result
    then stacks only those heads' rows, in the order given.
    """
    B, H, nq, nk, _ = shape
    ids = range(B * H) if heads is None else heads
    ids = list(ids)
    out = torch.empty(len(ids) * nq, nk, dtype=torch.bfloat16)
    for n, flat in enumerate(ids):
        out[n * nq:(n + 1) * nq] = causal_head(flat // H, flat % H, seed, shape)
    return out


WORKLOADS = {
    "normal_f32_128x781": Workload("normal_f32_128x781", "f32", 128, 781,
                                   "x ~ N(0,1), numpy PCG64 seed 0"),
    "normal_bf16_4096x4096": Workload("normal_bf16_4096x4096", "bf16", 4096, 4096,
                                      "x ~ N(0, 2^2), numpy PCG64 seed 2026, cast RNE"),
    **{f"spiky_f16_8192x{n}": Workload(f"spiky_f16_8192x{n}", "f16", 8192, n,
                                       "x ~ U(-8,8), 1% -> +/-1e4, seed 2026 per width")
       for n in SPIKE_WIDTHS},
    "offset_bf16_64x131072": Workload("offset_bf16_64x131072", "bf16", 64, 131072,
                                      "x ~ N(0,1) + row offset ~ U(-50,50), seed 2026"),
    "causal_bf16_524288x2048": Workload("causal_bf16_524288x2048", "bf16", 524288, 2048,
                                        "q.k^T/sqrt(128), causal -inf, seed (2026,b,h)"),
}


def generate(name: str) -> torch.Tensor:
    """Build a named workload on the CPU (the causal one takes a few seconds)."""
    if name == "normal_f32_128x781":
        return normal_f32_128x781()
    if name == "normal_bf16_4096x4096":
        return normal_bf16_4096x4096()
    if name.startswith("spiky_f16_8192x"):
        return spiky_f16(int(name.rsplit("x", 1)[1]))
    if name == "offset_bf16_64x131072":
        return offset_bf16_64x131072()
    if name == "causal_bf16_524288x2048":
        return causal_bf16()
    raise KeyError(name)


def upstream_grad(shape, dtype: str, seed: int = 7, device="cpu") -> torch.Tensor:
    """A seeded upstream gradient dy ~ N(0, 1) of ``shape``, rounded to ``dtype``, drawn
    by torch's generator on ``device`` (the backward's second input; a GPU generator
    makes the multi-GiB shapes without a host round trip)."""
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(_TORCH[dtype])


def storage_numpy(t: torch.Tensor) -> np.ndarray:
    """A CPU tensor's stored elements as numpy: float32, or the raw uint16 patterns of
    FP16/BF16 (a view, no conversion). Row-strided views stay views."""
    t = t.detach()
    if t.is_cuda:
        raise ValueError("expected a CPU tensor")
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(storage_numpy(t.contiguous()).tobytes()).hexdigest()
