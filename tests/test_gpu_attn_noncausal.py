"""GPU parity of attn_fwd / attn_bwd with causal = 0 (every token of a
document sees the whole document; no causal bound) against the fp64 oracle
with the same mask.

Tolerances as for the causal kernels: fp32 max-abs <= 1e-4; bf16 O within
max(2e-2, one bf16 ulp of |ref|), LSE within 1e-3; bf16 gradients within
max(2e-2, one bf16 ulp of |ref|), the same gradients with fp32 outputs within
2e-2, and the bf16 gradients equal to their round-to-nearest-even bit for bit.
"""
import numpy as np
import pytest
import torch

import sequence_parallelism_ulysses_amd as uly
import synthetic as syn
from oracle import attn_ref
from harness import DEV, Run, assert_close, bf16_tol, decode, dev_to_bits, sample_rows

pytestmark = pytest.mark.gpu


def run_noncausal(run, backward=True):
    c = run.cfg
    q, k, v = run.packed("q"), run.packed("k"), run.packed("v")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((c.hq, c.N), float("nan"), dtype=torch.float32, device=DEV)
    uly.attn_fwd(q, k, v, o, lse, c.scale, run.cu_dev, causal=0)
    out = dict(o=o, lse=lse)
    if backward:
        do = run.packed("do")
        ws = torch.empty(uly.attn_bwd_workspace_size(c.N, c.hq, c.hk, c.D, q.dtype), dtype=torch.uint8,
                         device=DEV)
        kinds = [("", q.dtype)] + ([("32", torch.float32)] if q.dtype == torch.bfloat16 else [])
        for suffix, gdt in kinds:
            g = {n: torch.full(t.shape, float("nan"), dtype=gdt, device=DEV) for n, t in (("dq", q), ("dk", k), ("dv", v))}
            bwd = uly.attn_bwd if gdt == q.dtype else uly.attn_bwd_ex
            bwd(q, k, v, o, do, lse, g["dq"], g["dk"], g["dv"], c.scale, ws, run.cu_dev, causal=0)
            out.update({n + suffix: t for n, t in g.items()})
    torch.cuda.synchronize()
    return out


def oracle(run, rows=None, backward=True):
    x = run.oracle_inputs()
    c = run.cfg
    return attn_ref(x["q"], x["k"], x["v"], c.scale, run.cu_host, do=x["do"] if backward else None,
                    rows=rows, causal=False)


def check(run, got, ref, rows=None, grads=True):
    c = run.cfg
    sel = slice(None) if rows is None else torch.from_numpy(rows).to(DEV)
    got_o = decode(dev_to_bits(got["o"][sel]))
    got_lse = got["lse"][:, sel].cpu().numpy().astype(np.float64)
    if c.dtype == "f32":
        assert_close(got_o, ref["o"], 1e-4, "O")
        assert_close(got_lse, ref["lse"], 1e-4, "LSE")
    else:
        assert_close(got_o, ref["o"], bf16_tol(ref["o"]), "O")
        assert_close(got_lse, ref["lse"], 1e-3, "LSE")
    if not grads:
        return
    names = ["dq"] if rows is not None else ["dq", "dk", "dv"]
    for n in names:
        if c.dtype == "f32":
            assert_close(decode(dev_to_bits(got[n][sel])), ref[n], 1e-4, n)
        else:
            g32 = got[n + "32"][sel]
            assert_close(g32.cpu().numpy().astype(np.float64), ref[n], 2e-2, n + " (fp32 out)")
            assert_close(decode(dev_to_bits(got[n][sel])), ref[n], bf16_tol(ref[n]), n)
            assert np.array_equal(dev_to_bits(got[n][sel]), dev_to_bits(g32.to(torch.bfloat16))), n


SMALL = [
    # N, P, Hq, Hkv, D, dtype, doc lengths (None = one document)
    (1000, 8, 32, 8, 128, "bf16", None),                          # ragged N, GQA 4:1
    (3000, 8, 32, 8, 128, "bf16", [1, 700, 0, 129, 1000, 1170]),  # packed docs, empty and 1-token docs
    (777, 7, 14, 14, 64, "bf16", None),                           # D=64, no GQA
    (512, 4, 32, 8, 128, "bf16", [64, 64, 128, 256]),             # tile-aligned documents
    (300, 2, 12, 4, 128, "bf16", [150, 150]),                     # G=3
    (333, 3, 6, 3, 128, "f32", None),                             # fp32 D=128
    (200, 2, 4, 2, 64, "f32", [33, 0, 167]),                      # fp32 D=64 with documents
    (8, 8, 8, 8, 128, "bf16", None),                              # fewer tokens than a tile
    (4096, 8, 32, 8, 128, "bf16", None),                          # many tiles, one document
]


@pytest.mark.parametrize("N,P,Hq,Hkv,D,dtype,lens", SMALL)
def test_noncausal_small_full(N, P, Hq, Hkv, D, dtype, lens):
    cfg = syn.custom(N, P, Hq, Hkv, D, dtype, seed=3 * N + D)
    cu = None if lens is None else syn.cu_from_lengths(lens)
    run = Run(cfg, cu=cu)
    check(run, run_noncausal(run), oracle(run))


def test_noncausal_c5_documents_sampled_rows():
    """The packed-document workload (65536 tokens, lognormal documents) with
    a document-only mask: O, LSE and dQ on sampled rows (document edges
    included), dK/dV through the document sum rules over every column."""
    cfg = syn.CONFIGS["c5"]
    run = Run(cfg)
    got = run_noncausal(run)
    rows = sample_rows(cfg.N, run.cu_host, n_random=96)
    check(run, got, oracle(run, rows=rows), rows=rows)
    # sum rules: sum_{j in doc} dK_j = 0 and sum_{j in doc} dV_j = sum_h sum_{i in doc} dO_{h,i}
    do = run.oracle_inputs(("do",))["do"]
    dk = got["dk32"].cpu().numpy().astype(np.float64)[:, 0]
    dv = got["dv32"].cpu().numpy().astype(np.float64)[:, 0]
    cu = np.asarray(run.cu_host)
    for a, b in zip(cu[:-1], cu[1:]):
        if a == b:
            continue
        rk = np.abs(dk[a:b].sum(axis=0)) / np.abs(dk[a:b]).sum(axis=0)
        rv = np.abs(dv[a:b].sum(axis=0) - do[a:b].sum(axis=(0, 1))) / np.abs(dv[a:b]).sum(axis=0)
        assert rk.max() < 1e-3 and rv.max() < 1e-3, (a, b, rk.max(), rv.max())


def test_causal_flag_changes_only_what_it_should():
    """Documents of one token: the causal and document-only masks agree, so
    both calls give the same bits."""
    N = 300
    cfg = syn.custom(N, 2, 8, 2, 128, "bf16", seed=9)
    run = Run(cfg, cu=syn.cu_from_lengths([1] * N))
    c = run.cfg
    q, k, v = run.packed("q"), run.packed("k"), run.packed("v")
    outs = []
    for causal in (1, 0):
        o = torch.empty_like(q)
        lse = torch.empty((c.hq, N), dtype=torch.float32, device=DEV)
        uly.attn_fwd(q, k, v, o, lse, c.scale, run.cu_dev, causal=causal)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
