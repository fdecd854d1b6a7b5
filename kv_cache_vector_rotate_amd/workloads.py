"""Seeded synthetic inputs for the key path (keys, queries).

This module generates inputs only; it holds none of the quantizer's
arithmetic, and both the HIP path and the CPU oracle consume its arrays.

Shapes follow the decode and cache workloads the pages measure on: a
Llama-3.1-8B-like decode step (32 query heads over 8 KV heads, head dim 128)
[Qiita explainer, benchmark models; ICLR 2026 digest, results table], a
Qwen2.5-3B-like full cache (36 layers x 2 KV heads, 8K context) [Qiita
explainer, community compression table], and a 1M-vector embedding index
[ICLR 2026 digest, vector-search results].  No benchmark data is used: keys
are z * scale with z ~ N(0,1), a per-(layer, KV-head) channel scale
exp(N(0, variance 0.5)) and four outlier channels multiplied by 20; queries
are N(0,1).  The search vectors use a per-dimension scale and are normalised
to unit length in float64 before the cast to float32.

Every (layer, KV head, batch) group draws from its own numpy Generator
seeded with a fixed tuple, so any group can be regenerated alone.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "workload", "group_keys", "group_queries", "all_keys",
           "all_queries", "f32_to_bf16_bits", "bf16_bits_to_f32", "WORKLOADS"]


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    layers: int
    kv_heads: int
    q_heads: int          # query heads per layer
    batch: int
    ctx: int              # keys per group
    d: int
    bits: int
    m: int
    key_dtype: str        # "bf16" or "f32"
    outliers: bool
    unit_norm: bool

    @property
    def G(self) -> int:
        return self.layers * self.kv_heads * self.batch

    @property
    def N(self) -> int:
        return self.ctx

    @property
    def Qg(self) -> int:
        return self.q_heads // self.kv_heads

    def group_coords(self, g: int):
        """group index -> (layer, batch, kv head); g = (layer*batch + b)*kv + h."""
        h = g % self.kv_heads
        rest = g // self.kv_heads
        return rest // self.batch, rest % self.batch, h


WORKLOADS = {
    0: Workload(0, "single-head d=128 N=4096 Qg=4 b=3 fp32", 1, 1, 4, 1, 4096, 128, 3, 128, "f32", True, False),
    1: Workload(1, "llama3.1-8b-decode bs16 32q/8kv d=128 ctx8192 b=3 bf16", 1, 8, 32, 16, 8192, 128, 3, 128, "bf16", True, False),
    2: Workload(2, "long-context bs4 32q/8kv d=128 ctx131072 b=4 bf16", 1, 8, 32, 4, 131072, 128, 4, 128, "bf16", True, False),
    3: Workload(3, "qwen2.5-3b cache 36L x 2kv 16q d=128 ctx8192 bs1 bf16", 36, 2, 16, 1, 8192, 128, 3, 128, "bf16", True, False),
    4: Workload(4, "vector-search N=1048576 d=1024 b=4 256 queries fp32", 1, 1, 256, 1, 1 << 20, 1024, 4, 1024, "f32", False, True),
}


def workload(cfg: int, bits: Optional[int] = None, ctx: Optional[int] = None) -> Workload:
    wl = WORKLOADS[cfg]
    if bits is not None:
        wl = dataclasses.replace(wl, bits=bits)
    if ctx is not None:
        wl = dataclasses.replace(wl, ctx=ctx)
    return wl


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        u = u + np.uint32(0x7FFF) + lsb
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK4 = 16384   # vectors per independently seeded chunk in the search workload


def _channel_scale(wl: Workload, layer: int, kvh: int):
    rng = np.random.default_rng([1000 + wl.cfg, layer, kvh])
    scale = np.exp(rng.normal(0.0, math.sqrt(0.5), wl.d))
    if wl.outliers:
        ch = rng.choice(wl.d, 4, replace=False)
        scale[ch] *= 20.0
    return scale


def group_keys(wl: Workload, g: int, start: int = 0, count: Optional[int] = None) -> np.ndarray:
    """Keys of group g, rows [start, start+count), as float32 values that are
    exact in the workload's key dtype (bf16-rounded for bf16 workloads)."""
    count = wl.N - start if count is None else count
    if wl.unit_norm:
        return _search_vectors(wl, start, count)
    layer, b, h = wl.group_coords(g)
    scale = _channel_scale(wl, layer, h)
    rng = np.random.default_rng([1000 + wl.cfg, layer, h, b + 1])
    z = rng.standard_normal((wl.N, wl.d), dtype=np.float32)
    k = (z[start:start + count] * scale.astype(np.float32)[None, :]).astype(np.float32)
    if wl.key_dtype == "bf16":
        k = bf16_bits_to_f32(f32_to_bf16_bits(k))
    return k


def _search_vectors(wl: Workload, start: int, count: int) -> np.ndarray:
    rng0 = np.random.default_rng([1000 + wl.cfg, 0])
    scale = np.exp(rng0.normal(0.0, math.sqrt(0.5), wl.d))
    out = np.empty((count, wl.d), dtype=np.float32)
    c0, c1 = start // _CHUNK4, (start + count - 1) // _CHUNK4
    for c in range(c0, c1 + 1):
        rng = np.random.default_rng([1000 + wl.cfg, 1, c])
        z = rng.standard_normal((_CHUNK4, wl.d)) * scale[None, :]
        z /= np.sqrt(np.sum(z * z, axis=1, keepdims=True))
        lo, hi = max(start, c * _CHUNK4), min(start + count, (c + 1) * _CHUNK4)
        out[lo - start:hi - start] = z[lo - c * _CHUNK4:hi - c * _CHUNK4].astype(np.float32)
    return out


def group_queries(wl: Workload, g: int) -> np.ndarray:
    """Queries [Qg, d] of group g (query head h of KV head k is h = k*Qg + j)."""
    layer, b, h = wl.group_coords(g)
    rng = np.random.default_rng([2000 + wl.cfg, layer, b])
    q = rng.standard_normal((wl.q_heads, wl.d), dtype=np.float32)
    q = q[h * wl.Qg:(h + 1) * wl.Qg]
    if wl.key_dtype == "bf16":
        q = bf16_bits_to_f32(f32_to_bf16_bits(q))
    return np.ascontiguousarray(q)


def all_keys(wl: Workload, groups=None) -> np.ndarray:
    """[len(groups), N, d] keys: uint16 bf16 bits for bf16 workloads, else float32."""
    groups = range(wl.G) if groups is None else groups
    groups = list(groups)
    dt = np.uint16 if wl.key_dtype == "bf16" else np.float32
    out = np.empty((len(groups), wl.N, wl.d), dtype=dt)
    for i, g in enumerate(groups):
        k = group_keys(wl, g)
        out[i] = f32_to_bf16_bits(k) if wl.key_dtype == "bf16" else k
    return out


def all_queries(wl: Workload, groups=None) -> np.ndarray:
    """[len(groups), Qg, d] queries in the same storage convention as keys."""
    groups = range(wl.G) if groups is None else groups
    groups = list(groups)
    dt = np.uint16 if wl.key_dtype == "bf16" else np.float32
    out = np.empty((len(groups), wl.Qg, wl.d), dtype=dt)
    for i, g in enumerate(groups):
        q = group_queries(wl, g)
        out[i] = f32_to_bf16_bits(q) if wl.key_dtype == "bf16" else q
    return out
