"""Seeded synthetic workloads shaped like the pages' experiments.

This module holds only input generation (random draws, outlier channels, unit-norm
scaling of database vectors).  It contains none of the codec's arithmetic, so both the
HIP path and the CPU oracle can be fed the same bytes from it.

Workload shapes (the pages' own models are not available; these stand in for them):
  * single_head   -- one head, d = 128, 1024 fp32 N(0,1) keys/values with 4 channels x20.
  * esm2_650m     -- 33 layers x 20 heads x d 64, 1024 tokens, bf16 Student-t (nu = 3),
                     3 per-head outlier channels x15, RoPE base 10000 ([TurboESM] section 3
                     reports ESM-2 650M, 33 layers, 20 heads, 1024 tokens).
  * llama3_8b     -- 32 layers, 32 q-heads / 8 kv-heads, d 128, batch 16, 32768 tokens,
                     bf16 N(0,1) with 3 channels (2% of 128) x10 per (layer, kv-head),
                     RoPE base 500000.
  * long_context  -- 1 layer, 64 q-heads / 8 kv-heads, d 128, batch 4, 131072 tokens,
                     bf16 unit-variance Laplace with 4 channels x20, RoPE base 500000;
                     the last 4096 positions are the timed append.
  * vector_search -- 10^6 database vectors of dimension 1536, fp32 N(0,1) scaled to unit
                     length, 1024 unit queries (stands in for the GloVe search experiment
                     of the TurboQuant summary, which is not available here).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    layers: int
    batch: int
    q_heads: int
    kv_heads: int
    d: int
    context: int          # tokens in the cache when the query attends
    bits_k: int
    bits_v: int
    m: int
    rope_base: float
    dtype: str            # "f32" | "bf16"
    dist: str             # "normal" | "student_t3" | "laplace"
    outliers: int
    outlier_scale: float
    append: int = 0       # tokens appended in one timed step (0: none)

    @property
    def q_pos(self) -> int:
        return self.context

    def scaled(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class SearchWorkload:
    name: str
    n_db: int
    nq: int
    d: int
    bits: int
    m: int
    k: int = 10

    def scaled(self, **kw) -> "SearchWorkload":
        return dataclasses.replace(self, **kw)


SINGLE_HEAD = DecodeWorkload("single_head", 1, 1, 1, 1, 128, 1024, 2, 3, 128, 0.0, "f32",
                             "normal", 4, 20.0)
ESM2_650M = DecodeWorkload("esm2_650m", 33, 1, 20, 20, 64, 1024, 2, 3, 64, 10000.0, "bf16",
                           "student_t3", 3, 15.0)
LLAMA3_8B = DecodeWorkload("llama3_8b", 32, 16, 32, 8, 128, 32768, 2, 3, 128, 500000.0, "bf16",
                           "normal", 3, 10.0)
LONG_CONTEXT = DecodeWorkload("long_context", 1, 4, 64, 8, 128, 131072, 2, 3, 128, 500000.0,
                              "bf16", "laplace", 4, 20.0, append=4096)
VECTOR_SEARCH = SearchWorkload("vector_search", 1_000_000, 1024, 1536, 3, 1536)

DECODE_WORKLOADS = {w.name: w for w in (SINGLE_HEAD, ESM2_650M, LLAMA3_8B, LONG_CONTEXT)}


def _seed(*parts) -> int:
    h = hashlib.sha256(("/".join(str(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & 0x7FFFFFFFFFFFFFFF


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def _draw(dist: str, shape, gen: torch.Generator, device) -> torch.Tensor:
    if dist == "normal":
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if dist == "student_t3":
        # Z / sqrt(chi2_3 / 3), chi2_3 as a sum of three squared normals (raw, variance 3)
        z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        c = torch.randn((3,) + tuple(shape), generator=gen, device=device, dtype=torch.float32)
        return z / torch.sqrt((c * c).sum(0) / 3.0)
    if dist == "laplace":
        # unit variance: scale 1/sqrt(2), as the difference of two exponentials
        u = torch.rand((2,) + tuple(shape), generator=gen, device=device, dtype=torch.float32)
        u = u.clamp_min(2.0 ** -30)
        return (torch.log(u[1]) - torch.log(u[0])) * float(1.0 / np.sqrt(2.0))
    raise ValueError(dist)


def outlier_channels(w: DecodeWorkload, layer: int, kv_head: int, seed: int = 0) -> np.ndarray:
    """Channel indices scaled by w.outlier_scale for one (layer, kv-head) unit.

    The single-head workload uses one fixed set; the multi-head ones pick per
    (layer, kv-head)."""
    rng = np.random.default_rng(_seed("outliers", w.name, seed, layer, kv_head))
    return np.sort(rng.choice(w.d, size=w.outliers, replace=False))


def gen_kv(w: DecodeWorkload, layer: int = 0, *, device="cpu", seed: int = 0, tokens=None):
    """K, V of shape [batch][kv_heads][tokens][d] in the workload's dtype.

    The same outlier channels are scaled in K and V of a unit."""
    T = w.context if tokens is None else tokens
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed("kv", w.name, seed, layer))
    shape = (w.batch, w.kv_heads, T, w.d)
    K = _draw(w.dist, shape, gen, device)
    V = _draw(w.dist, shape, gen, device)
    if w.outliers:
        scale = torch.ones((w.kv_heads, w.d), dtype=torch.float32)
        for h in range(w.kv_heads):
            scale[h, outlier_channels(w, layer, 0 if w.name == "single_head" else h, seed)] = w.outlier_scale
        scale = scale.to(device)[None, :, None, :]
        K.mul_(scale)
        V.mul_(scale)
    dt = _torch_dtype(w.dtype)
    return K.to(dt).contiguous(), V.to(dt).contiguous()


def gen_q(w: DecodeWorkload, layer: int = 0, *, device="cpu", seed: int = 0):
    """Queries [batch][q_heads][d] from the workload's base distribution, no outliers."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed("q", w.name, seed, layer))
    q = _draw(w.dist, (w.batch, w.q_heads, w.d), gen, device)
    return q.to(_torch_dtype(w.dtype)).contiguous()


def gen_search(w: SearchWorkload, *, device="cpu", seed: int = 0, chunk: int = 1 << 17):
    """(database [n_db][d], queries [nq][d]) fp32, rows scaled to unit length."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed("db", w.name, seed))
    db = torch.empty((w.n_db, w.d), dtype=torch.float32, device=device)
    for s in range(0, w.n_db, chunk):
        e = min(w.n_db, s + chunk)
        x = torch.randn((e - s, w.d), generator=gen, device=device, dtype=torch.float32)
        db[s:e] = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
    gq = torch.Generator(device=device)
    gq.manual_seed(_seed("queries", w.name, seed))
    q = torch.randn((w.nq, w.d), generator=gq, device=device, dtype=torch.float32)
    q = q / torch.linalg.vector_norm(q, dim=1, keepdim=True)
    return db, q
