"""Seeded synthetic inputs for the DDTree round (draws only, no method arithmetic).

This module is shared by the tests, the benchmark and the smoke check; it
feeds the same host tensors to the GPU path and to the CPU oracle. It holds
random draws and sizes, nothing that computes a step of the method.

Workloads stand in for the pages' evaluation data, which is not available:
drafter logits ~ N(0, sigma) per position with an optional planted token
boosted by a margin (a peaked drafter), target logits ~ N(0, sigma), and
Q/K/V ~ N(0, 1). Every draw uses torch's CPU generator seeded per workload,
so the inputs are identical on every machine.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    L: int              # draft block length = per-position distributions = max depth
    V: int              # vocabulary
    K: int              # per-position candidates
    N: int              # node budget (drafted nodes, root excluded)
    dtype: str          # "bf16" or "f32" for logits and Q/K/V
    logit_sigma: float
    boost: float        # planted-token margin at depth 1 (0 = none)
    boost_decay: bool   # margin decays linearly to 0 at depth L
    taus: Tuple[float, ...]
    Hq: int
    Hkv: int
    D: int
    prefix: Tuple[int, int]   # inclusive range of prefix lengths (lo == hi: fixed)
    target_sigma: float
    seed: int

    @property
    def T(self) -> int:
        return self.N + 1

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_L4_V64_K4_N8_P16", 1, 4, 64, 4, 8, "f32", 2.0, 0.0, False, (1.0,),
                 2, 2, 32, (16, 16), 2.0, 0),
        Workload("L16_V32000_K8_N64_P2048", 1, 16, 32000, 8, 64, "bf16", 3.0, 8.0, False,
                 (1.0,), 32, 8, 128, (2048, 2048), 3.0, 1),
        Workload("L16_V151936_K16_N256_P8192", 1, 16, 151936, 16, 256, "bf16", 3.0, 8.0, False,
                 (1.0, 0.0), 32, 8, 128, (8192, 8192), 3.0, 2),
        Workload("B32_L16_V151936_K8_N128_P512-16384", 32, 16, 151936, 8, 128, "bf16", 3.0, 8.0,
                 False, (1.0,), 32, 8, 128, (512, 16384), 3.0, 3),
        Workload("B4_L32_V151936_K16_N512_P65536", 4, 32, 151936, 16, 512, "bf16", 3.0, 8.0, True,
                 (1.0,), 64, 8, 128, (65536, 65536), 3.0, 4),
    ]
}
# The five workloads in order: tiny, then the four full-size ones.
WORKLOAD_ORDER = list(WORKLOADS)


def gen(seed: int) -> torch.Generator:
    return torch.Generator(device="cpu").manual_seed(int(seed))


def drafter_logits(w: Workload, seed: Optional[int] = None):
    """[batch, L, V] logits and the planted token per (request, position) (or None)."""
    g = gen(w.seed if seed is None else seed)
    out = torch.empty(w.batch, w.L, w.V, dtype=w.torch_dtype)
    planted = None
    if w.boost > 0:
        planted = torch.randint(0, w.V, (w.batch, w.L), generator=g)
    for b in range(w.batch):
        x = torch.randn(w.L, w.V, generator=g) * w.logit_sigma
        if planted is not None:
            for i in range(w.L):
                margin = w.boost
                if w.boost_decay and w.L > 1:
                    margin = w.boost * (1.0 - i / (w.L - 1))
                x[i, planted[b, i]] += margin
        out[b] = x.to(w.torch_dtype)
    return out, planted


def root_tokens(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    g = gen((w.seed if seed is None else seed) + 1000)
    return torch.randint(0, w.V, (w.batch,), generator=g, dtype=torch.int32)


def prefix_lengths(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    lo, hi = w.prefix
    if lo == hi:
        return torch.full((w.batch,), lo, dtype=torch.int32)
    g = gen((w.seed if seed is None else seed) + 2000)
    return torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int32)


def kv_offsets(prefix_lens: torch.Tensor, T: int) -> torch.Tensor:
    """Request b's KV rows start after all earlier requests' prefix+tree rows."""
    rows = prefix_lens.to(torch.int64) + T
    offs = torch.zeros_like(rows)
    if rows.numel() > 1:
        offs[1:] = torch.cumsum(rows, 0)[:-1]
    return offs


def qkv(w: Workload, prefix_lens: torch.Tensor, seed: Optional[int] = None, T: Optional[int] = None):
    """Q [batch, T, Hq, D]; K, V packed [sum_b (P_b + T), Hkv, D], ~N(0, 1)."""
    T = w.T if T is None else T
    g = gen((w.seed if seed is None else seed) + 3000)
    total = int(prefix_lens.to(torch.int64).sum().item()) + w.batch * T
    q = torch.randn(w.batch, T, w.Hq, w.D, generator=g).to(w.torch_dtype)
    k = torch.empty(total, w.Hkv, w.D, dtype=w.torch_dtype)
    v = torch.empty(total, w.Hkv, w.D, dtype=w.torch_dtype)
    step = 1 << 16
    for s in range(0, total, step):
        e = min(total, s + step)
        k[s:e] = torch.randn(e - s, w.Hkv, w.D, generator=g).to(w.torch_dtype)
        v[s:e] = torch.randn(e - s, w.Hkv, w.D, generator=g).to(w.torch_dtype)
    return q, k, v


def target_logits(w: Workload, seed: Optional[int] = None, T: Optional[int] = None) -> torch.Tensor:
    """[batch, T, V] target logits ~ N(0, target_sigma), one row per tree node."""
    T = w.T if T is None else T
    g = gen((w.seed if seed is None else seed) + 4000)
    out = torch.empty(w.batch, T, w.V, dtype=w.torch_dtype)
    for b in range(w.batch):
        out[b] = (torch.randn(T, w.V, generator=g) * w.target_sigma).to(w.torch_dtype)
    return out
