"""Seeded synthetic inputs for Fathom's read path.

This module only draws random numbers: keys, queries, budgets and the
fixed-width baseline's per-key side stream, with the shapes of the pages'
workload (Qwen3-8B: 36 layers, 8 KV heads, head dim 128, 32 query heads,
GQA group 4; up to 1M tokens).  It holds none of the method's arithmetic and
serves both the HIP path and the CPU oracle, which receive the same bytes.

Recipe (per configuration seed, layer and kv head):
  * channel scale sigma_c = exp(U(ln 0.1, ln 4)), log-uniform in [0.1, 4];
  * for the Qwen3-shaped workloads, 4 distinct outlier channels per kv head
    with sigma = 16 (chosen by a seeded random permutation);
  * key k[i, h, c] = sigma_c * N(0, 1); fp16 workloads round to fp16 (RN);
  * query q[h, c] ~ N(0, 1) in fp32;
  * budgets B: a fixed value, or drawn uniformly from a set per session.
Random streams come from torch's seeded generators on the requested device,
so the same seed gives the same bytes on the same kind of device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n: int                 # keys per session (tokens)
    hkv: int = 8
    hq: int = 32
    d: int = 128
    dtype: torch.dtype = torch.float16
    budget: int = 92       # bits per key per query head
    k: int = 2048
    outliers: int = 4
    seed: int = 1001
    layers: int = 1
    sessions: int = 1
    budget_set: tuple = field(default_factory=tuple)  # per-session B choices
    n_range: tuple = field(default_factory=tuple)     # ragged session lengths


# The five workloads.  Names say what they are; sizes follow the pages'
# Qwen3-8B, 1M-token single-GPU decode setting.
SINGLE_HEAD_4K = Workload("single-head d128 n4096 fp32 B92 k64", n=4096, hkv=1,
                          hq=1, dtype=torch.float32, budget=92, k=64,
                          outliers=0, seed=1001)
LAYER_128K = Workload("qwen3-8b layer n131072 fp16 k1024 hbm", n=131072,
                      budget=92, k=1024, seed=1002)
LAYER_1M = Workload("qwen3-8b layer n1048576 fp16 B92 k2048", n=1 << 20,
                    budget=92, k=2048, seed=1003)
SESSIONS_16 = Workload("16 ragged sessions n64K-512K fp16 k1024", n=0, k=1024,
                       seed=1004, sessions=16, budget_set=(68, 92, 136),
                       n_range=(65536, 524288))
STEP_36L_1M = Workload("qwen3-8b 36-layer decode step n1048576 B92 k2048",
                       n=1 << 20, budget=92, k=2048, seed=1005, layers=36)


def _cpu_gen(*parts: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    s = 0
    for p in parts:
        s = (s * 1000003 + int(p)) % (1 << 62)
    g.manual_seed(s)
    return g


def _dev_gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    s = 0
    for p in parts:
        s = (s * 1000003 + int(p)) % (1 << 62)
    g.manual_seed(s)
    return g


def channel_sigmas(seed: int, layer: int, hkv: int, d: int, outliers: int):
    """[hkv][d] fp64 channel scales (CPU)."""
    g = _cpu_gen(seed, layer, 1)
    u = torch.rand((hkv, d), generator=g, dtype=torch.float64)
    sig = torch.exp(math.log(0.1) + u * (math.log(4.0) - math.log(0.1)))
    for h in range(hkv):
        if outliers:
            perm = torch.randperm(d, generator=g)[:outliers]
            sig[h, perm] = 16.0
    return sig


def keys(seed: int, layer: int, n: int, hkv: int, d: int, dtype, outliers: int,
         device="cpu", session: int = 0) -> torch.Tensor:
    """Token-major keys [n][hkv][d] of the given dtype on ``device``."""
    sig = channel_sigmas(seed * 131 + session, layer, hkv, d, outliers)
    g = _dev_gen(device, seed, layer, session, 2)
    z = torch.randn((n, hkv, d), generator=g, device=device, dtype=torch.float32)
    z.mul_(sig.to(device=device, dtype=torch.float32).unsqueeze(0))
    return z.to(dtype)


def drifting_keys(seed: int, layer: int, n: int, hkv: int, d: int, dtype, outliers: int,
                  drift: float = 3.0, device="cpu", session: int = 0) -> torch.Tensor:
    """Keys of a long session whose ranges drift: keys() scaled per token by
    1 + drift * i / n and shifted by drift * sigma_c * u_c * i / n, with u_c
    ~ N(0, 1) per (kv head, channel).  The last token's range is about
    (1 + drift) times the first's, and centred elsewhere."""
    z = keys(seed, layer, n, hkv, d, torch.float32, outliers, device, session)
    sig = channel_sigmas(seed * 131 + session, layer, hkv, d, outliers)
    g = _cpu_gen(seed, layer, session, 8)
    u = torch.randn((hkv, d), generator=g, dtype=torch.float64)
    ramp = torch.arange(n, device=device, dtype=torch.float32) * (drift / max(n, 1))
    shift = (sig * u).to(device=device, dtype=torch.float32)
    z.mul_((1.0 + ramp)[:, None, None]).add_(ramp[:, None, None] * shift[None])
    return z.to(dtype)


def queries(seed: int, layer: int, hq: int, d: int, device="cpu",
            session: int = 0) -> torch.Tensor:
    g = _cpu_gen(seed, layer, session, 3)
    return torch.randn((hq, d), generator=g, dtype=torch.float32).to(device)


def side_stream(seed: int, layer: int, hkv: int, n: int, device="cpu",
                session: int = 0) -> torch.Tensor:
    """The fixed-width baseline's 8-bit per-key metadata [hkv][n] (uint8)."""
    g = _dev_gen(device, seed, layer, session, 4)
    return torch.randint(0, 256, (hkv, n), generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)


def side_stream4(seed: int, layer: int, hkv: int, n: int, device="cpu",
                 session: int = 0) -> torch.Tensor:
    """The r = 16 baseline's 4-bit per-key metadata, packed two keys per byte
    (even key in the low nibble): uint8 [hkv][ceil(n/2)], uniform bytes."""
    g = _dev_gen(device, seed, layer, session, 9)
    return torch.randint(0, 256, (hkv, (n + 1) // 2), generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)


def session_lengths(w: Workload):
    g = _cpu_gen(w.seed, 5)
    lo, hi = w.n_range
    return [int(v) for v in torch.randint(lo, hi + 1, (w.sessions,), generator=g)]


def session_budgets(w: Workload):
    g = _cpu_gen(w.seed, 6)
    idx = torch.randint(0, len(w.budget_set), (w.sessions,), generator=g)
    return [int(w.budget_set[int(i)]) for i in idx]


def random_budgets(seed: int, hq: int, lo: int, hi: int):
    g = _cpu_gen(seed, 7)
    return [int(v) for v in torch.randint(lo, hi + 1, (hq,), generator=g)]
