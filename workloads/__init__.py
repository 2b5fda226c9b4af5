"""Seeded synthetic inputs for jagged attention (shared by tests, bench and smoke).

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Values are drawn as float32 N(0, 1) with numpy's PCG64
``default_rng(seed)`` and rounded to bfloat16 with round-to-nearest-even (torch's
``.to(torch.bfloat16)``).  The draw order is: sequence lengths, then Q, K, V, G.

The five named workloads stand in for the pages' production shapes (batch 1152,
4 heads, head dim 128, sequences up to about 4k tokens), which are not public.
``rope_inputs`` lays out the rotary-embedding tables and positions that the fused
rotary backward takes as inputs.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

_CHUNK = 1 << 26  # elements per generation chunk (bounds host memory)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    broadcast_q: bool
    causal: bool
    batch: int
    heads: int
    head_dim: int
    q_len: int                 # broadcast query length (0 in self mode)
    lengths: tuple             # recipe: (kind, *params)
    offsets_dtype: str = "int32"
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    "tiny_broadcast": Workload(
        "tiny_broadcast", True, False, 4, 2, 64, 64, ("uniform", 1, 256), "int64",
        "broadcast-Q, B=4, H=2, D=64, Lq=64, KV lengths uniform in [1,256]"),
    "gem_broadcast": Workload(
        "gem_broadcast", True, False, 1152, 4, 128, 256, ("lognormal", 600.0, 1.0, 16, 4096), "int32",
        "GEM-shaped broadcast-Q, B=1152, H=4, D=128, Lq=256, KV lengths log-normal "
        "(median 600, sigma 1.0) clipped to [16,4096]"),
    "dq_stress": Workload(
        "dq_stress", True, False, 4096, 2, 128, 512, ("uniform", 32, 512), "int32",
        "dQ-contention stress, broadcast-Q, B=4096, H=2, D=128, Lq=512, KV lengths uniform in [32,512]"),
    "self_causal": Workload(
        "self_causal", False, True, 512, 8, 128, 0, ("zipf", 1.2, 64, 4096), "int32",
        "jagged causal self-attention, B=512, H=8, D=128, lengths Zipf(1.2) clipped to [64,4096]"),
    "block64": Workload(
        "block64", False, False, 36864, 4, 128, 0, ("fixed", 64), "int32",
        "block-diagonal attention: 1152 rows of 2048 tokens in 64-token blocks, H=4, D=128"),
}

ORDER = ["tiny_broadcast", "gem_broadcast", "dq_stress", "self_causal", "block64"]


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.lengths[0]
    if kind == "uniform":
        lo, hi = w.lengths[1], w.lengths[2]
        return rng.integers(lo, hi + 1, size=w.batch).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = w.lengths[1:]
        x = rng.lognormal(math.log(median), sigma, size=w.batch)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    if kind == "zipf":
        a, lo, hi = w.lengths[1:]
        return np.clip(rng.zipf(a, size=w.batch), lo, hi).astype(np.int64)
    if kind == "fixed":
        return np.full(w.batch, w.lengths[1], dtype=np.int64)
    raise ValueError(kind)


def offsets_from_lengths(lengths, dtype="int64") -> torch.Tensor:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return torch.from_numpy(off.astype(np.int32 if dtype == "int32" else np.int64))


def normal_bf16(rng: np.random.Generator, shape) -> torch.Tensor:
    """float32 N(0,1) draws rounded to bf16 (RNE), generated in bounded chunks."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16)
    pos = 0
    while pos < n:
        m = min(_CHUNK, n - pos)
        out[pos:pos + m] = torch.from_numpy(rng.standard_normal(m, dtype=np.float32)).to(torch.bfloat16)
        pos += m
    return out.view(*shape)


def normal_bf16_device(gen: torch.Generator, shape, device) -> torch.Tensor:
    """float32 N(0,1) draws from a seeded device generator, rounded to bf16 (RNE)."""
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_case(lengths, *, heads, head_dim, broadcast_q, causal=False, q_len=0, seed=0,
              offsets_dtype="int64", with_grad=True, rng=None, device=None):
    """Inputs for explicit sequence lengths.

    With device=None the values come from numpy (``rng`` or default_rng(seed)) and
    the tensors are on the CPU.  With a device, the values come from a torch
    generator on that device seeded with ``seed`` (fast at full size) and the
    tensors live there; offsets are always built from the lengths on the host.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    rows = len(lengths) * q_len if broadcast_q else total
    shapes = [(q_len if broadcast_q else total, heads, head_dim), (total, heads, head_dim),
              (total, heads, head_dim), (rows, heads, head_dim)]
    if device is None:
        rng = rng if rng is not None else np.random.default_rng(seed)
        draw = lambda shp: normal_bf16(rng, shp)  # noqa: E731
        offsets = offsets_from_lengths(lengths, offsets_dtype)
    else:
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        draw = lambda shp: normal_bf16_device(gen, shp, device)  # noqa: E731
        offsets = offsets_from_lengths(lengths, offsets_dtype).to(device)
    q = draw(shapes[0])
    k = draw(shapes[1])
    v = draw(shapes[2])
    g = draw(shapes[3]) if with_grad else None
    return dict(q=q, k=k, v=v, g=g, offsets=offsets,
                lengths=lengths, broadcast_q=broadcast_q, causal=causal,
                scale=1.0 / math.sqrt(head_dim), q_len=q_len if broadcast_q else 0)


def make_workload(name: str, seed: int = 0, with_grad: bool = True, offsets_dtype=None,
                  device=None):
    """The named workload at its full size (lengths first, then Q, K, V, G).

    Lengths always come from numpy default_rng(seed); values from the same numpy
    stream (device=None) or from a device generator seeded with ``seed``.
    """
    w = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(w, rng)
    case = make_case(lengths, heads=w.heads, head_dim=w.head_dim, broadcast_q=w.broadcast_q,
                     causal=w.causal, q_len=w.q_len, offsets_dtype=offsets_dtype or w.offsets_dtype,
                     with_grad=with_grad, rng=rng, seed=seed, device=device)
    case["workload"] = w
    return case


def rope_inputs(case, base: float = 10000.0):
    """Rotary-embedding inputs for a case: fp32 tables cos / sin of shape
    [max_pos, D/2] with angle p * base ** (-2 d / D) (the common frequency recipe,
    computed in fp64 and rounded to fp32), and int32 positions: every key row's
    index within its sequence, and every query row's (broadcast: 0 .. Lq - 1;
    self: the key positions).  CPU tensors."""
    lengths = np.asarray(case["lengths"], dtype=np.int64)
    d = case["k"].shape[2]
    pos_k = np.concatenate([np.arange(n, dtype=np.int64) for n in lengths]) if len(lengths) else \
        np.zeros(0, dtype=np.int64)
    pos_q = np.arange(case["q_len"], dtype=np.int64) if case["broadcast_q"] else pos_k
    max_pos = max(int(lengths.max()) if len(lengths) else 0, int(case["q_len"]), 1)
    inv = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return dict(cos=torch.from_numpy(np.cos(ang).astype(np.float32)),
                sin=torch.from_numpy(np.sin(ang).astype(np.float32)),
                pos_q=torch.from_numpy(pos_q.astype(np.int32)),
                pos_k=torch.from_numpy(pos_k.astype(np.int32)))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a bf16 (or any float) CPU tensor to a numpy fp64 array."""
    return t.to(torch.float64).numpy()
