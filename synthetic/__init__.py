"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU oracle.

This module only draws numbers: packed sequence lengths (``cu_seqlens``) and
N(0, 1) tensors.  It holds none of the attention arithmetic, so that the HIP
path and the oracle stay independent of each other.

Workloads (the pages measure on no public dataset; every input here is
synthetic and stands in for packed training batches):

* ``c1`` fp32, 256 tokens packed as [96, 64, 96], 2/2 heads, d=32, CP=2.
* ``c2`` bf16, 8192 tokens, lengths uniform in [128, 4096] rounded up to a
  multiple of 2*CP, 16/16 heads, d=128, CP=4.
* ``c3`` bf16, one causal sequence of 32768 tokens, GQA 32/8, d=128, CP=8.
* ``c4`` bf16, 65536 tokens, lengths log-uniform in [64, 16384] rounded up to
  a multiple of 16, GQA 64/8, d=128, CP=8.
* ``c5`` bf16, one causal sequence of 131072 tokens, GQA 64/8, d=128, CP=16,
  forward and backward.

Packing to an exact token budget: lengths are drawn, rounded up to the
multiple, and appended until the running sum reaches the budget; the last
length is cut to what is left (it stays a multiple, since the budget is one,
and may fall below the stated minimum).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "lengths_for", "cu_seqlens_for", "make_cu_seqlens",
    "lengths_uniform", "lengths_loguniform", "randn_qkv", "randn_qkv_device",
    "round_bf16", "random_lengths",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    total: int            # packed tokens T
    hq: int
    hkv: int
    d: int
    cp: int
    seed: int
    backward: bool
    lengths: Optional[tuple] = None   # fixed lengths, else drawn
    dist: str = "fixed"               # "fixed", "uniform", "loguniform"
    lo: int = 0
    hi: int = 0
    mult: int = 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "c1": Workload("c1", "f32", 256, 2, 2, 32, 2, 1, False, lengths=(96, 64, 96)),
    "c2": Workload("c2", "bf16", 8192, 16, 16, 128, 4, 2, False, dist="uniform",
                   lo=128, hi=4096, mult=8),
    "c3": Workload("c3", "bf16", 32768, 32, 8, 128, 8, 3, False, lengths=(32768,)),
    "c4": Workload("c4", "bf16", 65536, 64, 8, 128, 8, 4, False, dist="loguniform",
                   lo=64, hi=16384, mult=16),
    "c5": Workload("c5", "bf16", 131072, 64, 8, 128, 16, 5, True, lengths=(131072,)),
}


def _pack(draw, total: int, mult: int) -> List[int]:
    out: List[int] = []
    acc = 0
    while acc < total:
        L = int(draw())
        L = ((L + mult - 1) // mult) * mult
        L = min(L, total - acc)
        out.append(L)
        acc += L
    return out


def lengths_uniform(seed: int, total: int, lo: int, hi: int, mult: int) -> List[int]:
    rng = np.random.default_rng(seed)
    return _pack(lambda: rng.integers(lo, hi + 1), total, mult)


def lengths_loguniform(seed: int, total: int, lo: int, hi: int, mult: int) -> List[int]:
    rng = np.random.default_rng(seed)
    return _pack(lambda: round(math.exp(rng.uniform(math.log(lo), math.log(hi)))), total, mult)


def lengths_for(w: Workload) -> List[int]:
    if w.lengths is not None:
        return list(w.lengths)
    if w.dist == "uniform":
        return lengths_uniform(w.seed, w.total, w.lo, w.hi, w.mult)
    if w.dist == "loguniform":
        return lengths_loguniform(w.seed, w.total, w.lo, w.hi, w.mult)
    raise ValueError(w.dist)


def make_cu_seqlens(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def cu_seqlens_for(w: Workload) -> np.ndarray:
    return make_cu_seqlens(lengths_for(w))


def random_lengths(seed: int, nseq_max: int, chunk_max: int, cp: int) -> List[int]:
    """Small random packings for property tests: each length is a multiple of 2*cp."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, nseq_max + 1))
    return [int(rng.integers(1, chunk_max + 1)) * 2 * cp for _ in range(n)]


def round_bf16(x):
    """Round an fp32 torch tensor to bf16 (round to nearest even) and back to fp32."""
    import torch
    return x.to(torch.bfloat16).to(torch.float32)


def randn_qkv(seed: int, total: int, hq: int, hkv: int, d: int, dtype: str,
              with_do: bool = False, q_scale: float = 1.0):
    """CPU tensors Q, K, V (and dO), drawn N(0,1) in fp32 in that order from one
    generator, then cast to the workload dtype.  Layout [T, H, d]."""
    import torch
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((total, hq, d), generator=g, dtype=torch.float32)
    k = torch.randn((total, hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((total, hkv, d), generator=g, dtype=torch.float32)
    do = torch.randn((total, hq, d), generator=g, dtype=torch.float32) if with_do else None
    if q_scale != 1.0:
        q = q * q_scale
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = [q.to(tdt), k.to(tdt), v.to(tdt)]
    if with_do:
        out.append(do.to(tdt))
    return tuple(out)


def randn_qkv_device(seed: int, total: int, hq: int, hkv: int, d: int, dtype: str,
                     device, with_do: bool = False):
    """Same shapes and distribution as :func:`randn_qkv`, drawn on the device
    (fast for the largest workload; values differ from the CPU draw)."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    shapes = [(total, hq, d), (total, hkv, d), (total, hkv, d)]
    if with_do:
        shapes.append((total, hq, d))
    return tuple(torch.randn(s, generator=g, dtype=torch.float32, device=device).to(tdt)
                 for s in shapes)
