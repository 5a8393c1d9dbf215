"""attn_bwd_noalloc (the backward with the library's static device buffer as
workspace, for callers that cannot allocate) against attn_bwd on the same
inputs, on consecutive calls whose sizes shrink and whose types change: dq
bitwise, dk/dv (whose float32 sums run in another order) within the
attention bar, max(2e-2, one bf16 ulp of |x|), and 1e-4 for fp32. It also
checks that the calls take no device memory."""
import numpy as np
import pytest
import torch

import sequence_parallelism_ulysses_amd as uly
import synthetic as syn
from harness import DEV, Run, assert_close, bf16_tol, decode, dev_to_bits

pytestmark = pytest.mark.gpu

CASES = [
    # (N, P, Hq, Hkv, D, dtype, document lengths): the 32k Llama-3.1-8B head
    # group, then smaller inputs: packed documents, fp32
    (32768, 8, 32, 8, 128, "bf16", None),
    (3000, 8, 32, 8, 128, "bf16", [1, 700, 0, 129, 1000, 1170]),
    (1024, 4, 8, 8, 64, "f32", None),
]


def _inputs(case):
    N, P, Hq, Hkv, D, dtype, lens = case
    cfg = syn.custom(N, P, Hq, Hkv, D, dtype, seed=N + 17)
    run = Run(cfg, cu=None if lens is None else syn.cu_from_lengths(lens))
    q, k, v, do = run.packed("q"), run.packed("k"), run.packed("v"), run.packed("do")
    o = torch.empty_like(q)
    lse = torch.empty((cfg.hq, N), dtype=torch.float32, device=DEV)
    uly.attn_fwd(q, k, v, o, lse, cfg.scale, run.cu_dev)
    return cfg, run, (q, k, v, o, do, lse)


def _grads(t):
    q, k, v = t[0], t[1], t[2]
    return [torch.full(x.shape, float("nan"), dtype=x.dtype, device=DEV) for x in (q, k, v)]


def test_noalloc_matches_attn_bwd_on_consecutive_calls():
    prepared = [_inputs(c) for c in CASES]
    # reference: attn_bwd with a caller-provided workspace
    refs = []
    for cfg, run, t in prepared:
        ws = torch.empty(uly.attn_bwd_workspace_size(cfg.N, cfg.hq, cfg.hk, cfg.D, t[0].dtype), dtype=torch.uint8,
                         device=DEV)
        g = _grads(t)
        uly.attn_bwd(*t, *g, cfg.scale, ws, run.cu_dev)
        refs.append(g)
        del ws
    outs = [_grads(t) for _, _, t in prepared]
    torch.cuda.synchronize()
    for rep in range(2):
        for g in outs:
            for x in g:
                x.fill_(float("nan"))
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        for (cfg, run, t), g in zip(prepared, outs):  # largest first, then smaller ones
            uly.attn_bwd_noalloc(*t, *g, cfg.scale, run.cu_dev)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        if rep == 1:  # after the first repetition (module load), no device memory taken
            assert free1 >= free0, f"attn_bwd_noalloc took {free0 - free1} bytes of device memory"
        for (cfg, run, t), got, ref in zip(prepared, outs, refs):
            bits = (lambda x: x.view(torch.int16)) if got[0].dtype == torch.bfloat16 else (lambda x: x)
            assert torch.equal(bits(got[0]), bits(ref[0])), (cfg.workload, "dq differs")
            for name, a, b in (("dk", got[1], ref[1]), ("dv", got[2], ref[2])):
                x, y = decode(dev_to_bits(a)), decode(dev_to_bits(b))
                tol = 1e-4 if cfg.dtype == "f32" else bf16_tol(y)
                assert_close(x, y, tol, f"{cfg.workload} {name}")
                print(f"call {rep} {cfg.workload} {name}: max |noalloc - attn_bwd| = {np.abs(x - y).max():.3g}",
                      flush=True)


def test_noalloc_rejects_sizes_beyond_the_buffer():
    cfg = syn.custom(51784, 8, 32, 8, 128, "bf16", seed=1)
    q = torch.empty((cfg.N, cfg.hq, cfg.D), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((cfg.N, cfg.hk, cfg.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((cfg.hq, cfg.N), dtype=torch.float32, device=DEV)
    with pytest.raises(uly.UlyssesError) as e:
        uly.attn_bwd_noalloc(q, k, k, q, q, lse, q, k, k, cfg.scale)
    assert e.value.status == uly.ULY_ERR_UNSUPPORTED
