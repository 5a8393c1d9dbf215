"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the binding, and build the oracle's expectations.

The oracle side never sees a GPU result as an input: it packs the host shards
itself and computes attention from the decoded input values.
"""
from __future__ import annotations

import numpy as np
import torch

import sequence_parallelism_ulysses_amd as uly
import synthetic as syn
from oracle import attn_ref, bf16_bits_to_f64, f32_bits_to_f64, pack_ref

DEV = "cuda:0"


def torch_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(bits.view(np.float32)).to(DEV)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    raise TypeError(t.dtype)


def decode(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(bits) if bits.dtype == np.uint16 else f32_bits_to_f64(bits)


def bf16_tol(ref: np.ndarray, base: float = 2e-2) -> np.ndarray:
    """Element-wise bound max(base, one bf16 ulp of |ref|): a correctly rounded
    bf16 result can be off by half an ulp, which exceeds 2e-2 once |ref| >= 8."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    return np.maximum(base, np.exp2(e - 7))


def grad_tol(ref: np.ndarray, G: int, name: str) -> np.ndarray:
    """The bf16 gradient bar: bf16_tol(ref). dK and dV of a kv head sum the
    gradients of its G query heads, so their rounding errors add up over G
    independent terms; the 2e-2 bar is stated for the workloads' G = 4, and
    for larger G the base grows as sqrt(G / 4)."""
    base = 2e-2 * max(1.0, (G / 4) ** 0.5) if name in ("dk", "dv") else 2e-2
    return bf16_tol(ref, base)


def err_report(what: str, got: np.ndarray, ref: np.ndarray) -> str:
    """Max-abs error, max |ref|, the count of elements whose error exceeds
    2e-2, and the worst error relative to bf16_tol; printed and returned."""
    err = np.abs(got - ref)
    line = (f"{what}: max err {err.max():.4g}, max |ref| {np.abs(ref).max():.4g}, "
            f"{int((err > 2e-2).sum())} of {err.size} elements above 2e-2, "
            f"worst err / max(2e-2, ulp) = {(err / bf16_tol(ref)).max():.3f}")
    print(line, flush=True)
    return line


def assert_close(got: np.ndarray, ref: np.ndarray, tol, what: str):
    err = np.abs(got - ref)
    bad = err > tol
    if np.any(~np.isfinite(got)) or np.any(bad):
        idx = np.argwhere(bad | ~np.isfinite(got))[:5]
        raise AssertionError(f"{what}: max err {np.nanmax(err):.3g} (max |ref| {np.abs(ref).max():.3g}), "
                             f"{int(bad.sum())} elements over tolerance, first at {idx.tolist()}")


class Run:
    """Host shards + their device copies for one config."""

    def __init__(self, cfg, cu=None, tensors=("q", "k", "v", "do")):
        self.cfg = cfg
        self.cu_host = cu if cu is not None else syn.cu_seqlens(cfg)
        self.cu_dev = None if self.cu_host is None else torch.from_numpy(
            np.asarray(self.cu_host, dtype=np.int32)).to(DEV)
        self.host = {n: syn.all_shards_bits(cfg, n) for n in tensors}
        self.dev = {n: [bits_to_dev(s) for s in self.host[n]] for n in tensors}

    def packed(self, name: str) -> torch.Tensor:
        c = self.cfg
        sh = self.dev[name]
        out = torch.empty((c.N, c.group_heads(name), c.D), dtype=sh[0].dtype, device=DEV)
        uly.ulysses_pack(sh, c.group, out)
        return out

    def oracle_inputs(self, names=("q", "k", "v", "do")):
        return {n: decode(pack_ref(self.host[n], self.cfg.group)) for n in names if n in self.host}


def oracle_attention(run: Run, rows=None, backward=True):
    x = run.oracle_inputs()
    c = run.cfg
    return attn_ref(x["q"], x["k"], x["v"], c.scale, run.cu_host, do=x["do"] if backward else None, rows=rows)


def sample_rows(N: int, cu, n_random: int = 192, seed: int = 0) -> np.ndarray:
    """Query rows to check at sizes the full oracle cannot finish quickly:
    first/last rows, tile edges, document edges, and random rows."""
    r = np.random.default_rng(seed)
    s = {0, 1, N - 1, N - 2}
    for e in (31, 32, 63, 64, 127, 128, 255, 256, 4095, 4096, N // 2, N // 2 + 1):
        if e < N:
            s.add(e)
    if cu is not None:
        for b in np.asarray(cu)[1:-1]:
            for e in (b - 1, b, b + 1):
                if 0 <= e < N:
                    s.add(int(e))
    s.update(int(x) for x in r.integers(0, N, size=n_random))
    return np.array(sorted(s), dtype=np.int64)
