"""Seeded synthetic inputs for one GPU's share of Ulysses sequence parallelism.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds none of the method's arithmetic: only random draws, the rounding of those
draws to bf16 (which is how bf16 input values are made), and the sampling of
packed-document lengths. Neither the oracle nor the HIP path is imported here.

Workloads (one GPU's share; "Ulysses Sequence Parallelism: Training with
Million-Token Contexts", the sequence-sharding and all-to-all steps):

  c1  fp32, N=1024 split into P=4 shards of 256, 8 q heads = 8 kv heads, D=64,
      head group 0 (2 q heads, 2 kv heads), scale 1/8
  c2  bf16, N=32768, P=8, 32 q / 8 kv heads (Llama-3.1-8B attention shape),
      D=128, head group 0 -> 4 q heads sharing 1 kv head
  c3  as c2 at N=131072
  c4  as c2 at N=1048576
  c5  as c2 at N=65536 built from packed documents whose lengths are
      lognormal(mu=ln 4096, sigma=1) clipped to [128, 32768]

Every tensor is drawn shard by shard in the sequence-sharded layout
[T, H, D] (T = N/P tokens, H = all heads), one SeedSequence child per
(tensor, shard), so any single shard can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSORS = ("q", "k", "v", "do")
_BASE_SEED = 20260309


@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    workload: str
    N: int
    P: int
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32" or "bf16"
    group: int = 0
    varlen: bool = False
    seed: int = 0

    @property
    def T(self) -> int:
        return self.N // self.P

    @property
    def hq(self) -> int:
        return self.Hq // self.P

    @property
    def hk(self) -> int:
        return self.Hkv // self.P

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def heads(self, which: str) -> int:
        return self.Hq if which in ("q", "do", "o", "dq") else self.Hkv

    def group_heads(self, which: str) -> int:
        return self.heads(which) // self.P


def _cfg(idx: int, workload: str, **kw) -> Config:
    return Config(key=f"c{idx}", workload=workload, seed=_BASE_SEED + idx, **kw)


CONFIGS = {
    "c1": _cfg(1, "tiny-fp32-n1024-p4-h8-d64", N=1024, P=4, Hq=8, Hkv=8, D=64, dtype="f32"),
    "c2": _cfg(2, "llama3.1-8b-attn-n32768-p8-gqa32q8kv-d128", N=32768, P=8, Hq=32, Hkv=8, D=128, dtype="bf16"),
    "c3": _cfg(3, "llama3.1-8b-attn-n131072-p8-gqa32q8kv-d128", N=131072, P=8, Hq=32, Hkv=8, D=128, dtype="bf16"),
    "c4": _cfg(4, "llama3.1-8b-attn-n1048576-p8-gqa32q8kv-d128", N=1048576, P=8, Hq=32, Hkv=8, D=128, dtype="bf16"),
    "c5": _cfg(5, "packed-sft-n65536-lognormal-docs-p8-gqa32q8kv-d128", N=65536, P=8, Hq=32, Hkv=8, D=128, dtype="bf16", varlen=True),
}


def custom(N: int, P: int, Hq: int, Hkv: int, D: int, dtype: str, group: int = 0,
           varlen: bool = False, seed: int = 1) -> Config:
    """A config outside the five named workloads (ragged tails, edge cases)."""
    return Config(key="custom", workload=f"custom-n{N}-p{P}-h{Hq}-{Hkv}-d{D}-{dtype}",
                  N=N, P=P, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, group=group,
                  varlen=varlen, seed=seed)


# --------------------------------------------------------------------------
# bf16 encoding of draws (round to nearest, ties to even); inputs only.
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return uint16 bits.

    The draws are finite normals, so no NaN/Inf handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# shards
# --------------------------------------------------------------------------
def _seed_children(cfg: Config):
    ss = np.random.SeedSequence(cfg.seed)
    kids = ss.spawn(len(TENSORS) + 1)
    return {name: kids[i] for i, name in enumerate(TENSORS)}, kids[-1]


def shard_bits(cfg: Config, which: str, j: int, T: int | None = None) -> np.ndarray:
    """Raw bits of shard j of tensor `which` ("q","k","v","do"), shape [T, H, D].

    uint16 for bf16 configs, uint32 for fp32 configs. The values are N(0,1)
    draws (float32), rounded to bf16 for bf16 configs."""
    if which not in TENSORS:
        raise ValueError(which)
    if not 0 <= j < cfg.P:
        raise ValueError("shard index out of range")
    T = cfg.T if T is None else T
    tensor_seeds, _ = _seed_children(cfg)
    child = tensor_seeds[which].spawn(cfg.P)[j]
    rng = np.random.Generator(np.random.PCG64(child))
    x = rng.standard_normal((T, cfg.heads(which), cfg.D), dtype=np.float32)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x.view(np.uint32)


def shard_values(cfg: Config, which: str, j: int) -> np.ndarray:
    """The float32 values those bits encode (exact)."""
    bits = shard_bits(cfg, which, j)
    return bf16_bits_to_f32(bits) if cfg.dtype == "bf16" else bits.view(np.float32)


def all_shards_bits(cfg: Config, which: str) -> list[np.ndarray]:
    return [shard_bits(cfg, which, j) for j in range(cfg.P)]


# --------------------------------------------------------------------------
# packed documents
# --------------------------------------------------------------------------
def lognormal_doc_lengths(N: int, rng: np.random.Generator, mu: float = math.log(4096.0),
                          sigma: float = 1.0, lo: int = 128, hi: int = 32768) -> list[int]:
    """Document lengths L = clip(rint(exp(N(mu, sigma))), lo, hi), drawn until
    they cover N tokens; the last one is cut so the lengths sum to exactly N."""
    out: list[int] = []
    total = 0
    while total < N:
        L = int(np.clip(np.rint(np.exp(rng.normal(mu, sigma))), lo, hi))
        L = min(L, N - total)
        out.append(L)
        total += L
    return out


def cu_seqlens(cfg: Config) -> np.ndarray | None:
    """int32 document offsets [ndocs+1] (0 first, N last) for varlen configs,
    None (one document of N tokens) otherwise."""
    if not cfg.varlen:
        return None
    _, doc_seed = _seed_children(cfg)
    rng = np.random.Generator(np.random.PCG64(doc_seed))
    lens = lognormal_doc_lengths(cfg.N, rng)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)
