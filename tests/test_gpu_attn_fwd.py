"""GPU parity of attn_fwd (reached through ulysses_pack from seeded shards)
against the fp64 oracle.

Tolerances: fp32 workload max-abs <= 1e-4 (O and LSE); bf16 O within
max(2e-2, one bf16 ulp of |ref|) element-wise, LSE (fp32 output) within 1e-3.
"""
import numpy as np
import pytest
import torch

import sequence_parallelism_ulysses_amd as uly
import synthetic as syn
from harness import DEV, Run, assert_close, bf16_tol, dev_to_bits, decode, oracle_attention, sample_rows

pytestmark = pytest.mark.gpu


def run_fwd(run):
    c = run.cfg
    q, k, v = run.packed("q"), run.packed("k"), run.packed("v")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((c.hq, c.N), float("nan"), dtype=torch.float32, device=DEV)
    uly.attn_fwd(q, k, v, o, lse, c.scale, run.cu_dev)
    torch.cuda.synchronize()
    return o, lse


def check_fwd(run, rows=None):
    c = run.cfg
    o, lse = run_fwd(run)
    ref = oracle_attention(run, rows=rows, backward=False)
    sel = slice(None) if rows is None else torch.from_numpy(rows).to(DEV)
    got_o = decode(dev_to_bits(o[sel]))
    got_lse = lse[:, sel].cpu().numpy().astype(np.float64)
    if c.dtype == "f32":
        assert_close(got_o, ref["o"], 1e-4, "O")
        assert_close(got_lse, ref["lse"], 1e-4, "LSE")
    else:
        assert_close(got_o, ref["o"], bf16_tol(ref["o"]), "O")
        assert_close(got_lse, ref["lse"], 1e-3, "LSE")
    return o, lse


def test_fwd_c1_fp32_full():
    check_fwd(Run(syn.CONFIGS["c1"], tensors=("q", "k", "v")))


SMALL = [
    # N, P, Hq, Hkv, D, dtype, doc lengths (None = one document)
    (1000, 8, 32, 8, 128, "bf16", None),                       # ragged N, GQA 4:1
    (3000, 8, 32, 8, 128, "bf16", [1, 700, 0, 129, 1000, 1170]),  # packed docs, empty and 1-token docs
    (777, 7, 14, 14, 64, "bf16", None),                        # D=64, no GQA (2 heads, 2 kv heads)
    (512, 4, 32, 8, 128, "bf16", [64, 64, 128, 256]),          # 8 q heads over 2 kv heads, tile-aligned docs
    (300, 2, 12, 4, 128, "bf16", [150, 150]),                  # G=3: one q head per workgroup
    (333, 3, 6, 3, 128, "f32", None),                          # fp32 D=128, GQA 2:1
    (64, 1, 4, 1, 64, "f32", [10, 54]),                        # one tile, fp32 D=64
    (8, 8, 8, 8, 128, "bf16", None),                           # fewer tokens than a tile
    (1000, 4, 32, 4, 128, "bf16", None),                       # G=8: one 32-row tile, 8 heads per workgroup
    (1536, 2, 32, 2, 128, "bf16", [700, 836]),                 # G=16: two head groups per kv head
    (640, 1, 8, 1, 64, "bf16", [100, 1, 539]),                 # G=8, D=64
    (512, 2, 64, 4, 128, "bf16", None),                        # G=16 over two kv heads
]


@pytest.mark.parametrize("N,P,Hq,Hkv,D,dtype,lens", SMALL)
def test_fwd_small_full(N, P, Hq, Hkv, D, dtype, lens):
    cfg = syn.custom(N, P, Hq, Hkv, D, dtype, seed=N + D)
    cu = None if lens is None else syn.cu_from_lengths(lens)
    check_fwd(Run(cfg, cu=cu, tensors=("q", "k", "v")))


@pytest.mark.parametrize("key", ["c2", "c5"])
def test_fwd_workload_sampled_rows(key):
    cfg = syn.CONFIGS[key]
    run = Run(cfg, tensors=("q", "k", "v"))
    check_fwd(run, rows=sample_rows(cfg.N, run.cu_host))


def test_fwd_c3_sampled_rows():
    cfg = syn.CONFIGS["c3"]
    run = Run(cfg, tensors=("q", "k", "v"))
    check_fwd(run, rows=sample_rows(cfg.N, None, n_random=64))


@pytest.mark.parametrize("N,P,Hq,Hkv,D,lens,causal", [
    (32768, 8, 32, 8, 128, None, 1),            # the Llama-3.1-8B-shaped 32k head group
    (256, 4, 16, 4, 128, None, 1),              # one tile per shard
    (1024, 2, 8, 2, 64, [300, 1, 0, 723], 1),   # documents across the shard boundary, D = 64
    (768, 3, 12, 6, 128, [500, 268], 0),        # document-only mask, G = 2
])
def test_fwd_from_shards_equals_pack_then_fwd(N, P, Hq, Hkv, D, lens, causal):
    """Reading the sequence-sharded Q/K/V in place gives the bits that
    ulysses_pack + attn_fwd give (the same operands reach the same products),
    and matches the oracle."""
    cfg = syn.custom(N, P, Hq, Hkv, D, "bf16", group=P - 1, seed=N + Hq)
    cu = None if lens is None else syn.cu_from_lengths(lens)
    run = Run(cfg, cu=cu, tensors=("q", "k", "v"))
    q, k, v = run.packed("q"), run.packed("k"), run.packed("v")
    o1 = torch.empty_like(q)
    l1 = torch.empty((cfg.hq, N), dtype=torch.float32, device=DEV)
    uly.attn_fwd(q, k, v, o1, l1, cfg.scale, run.cu_dev, causal=causal)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((cfg.hq, N), float("nan"), dtype=torch.float32, device=DEV)
    uly.attn_fwd_from_shards(run.dev["q"], run.dev["k"], run.dev["v"], cfg.group, o2, l2, cfg.scale, run.cu_dev,
                             causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    rows = sample_rows(N, run.cu_host, n_random=64)
    x = run.oracle_inputs(("q", "k", "v"))
    from oracle import attn_ref
    ref = attn_ref(x["q"], x["k"], x["v"], cfg.scale, run.cu_host, rows=rows, causal=bool(causal))
    sel = torch.from_numpy(rows).to(DEV)
    assert_close(decode(dev_to_bits(o2[sel])), ref["o"], bf16_tol(ref["o"]), "O")
    assert_close(l2[:, sel].cpu().numpy().astype(np.float64), ref["lse"], 1e-3, "LSE")
