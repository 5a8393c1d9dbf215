"""GPU property tests of the attention kernels (no oracle): statements of the
method that hold bit for bit whatever the inputs.

  - causality: perturbing every token after position i0 leaves O, LSE and
    dQ of the rows up to i0 unchanged (masked keys contribute exact zeros);
  - document isolation: perturbing one packed document leaves every output
    of the other documents unchanged, gradients included;
  - GQA: q heads sharing a kv head give the same O and LSE as multi-head
    attention with that kv head repeated, and dK/dV equal to the sum of the
    repeated heads' gradients (to fp32 rounding).
"""
import numpy as np
import pytest
import torch

import sequence_parallelism_ulysses_amd as uly
from harness import DEV

pytestmark = pytest.mark.gpu


def _inputs(N, hq, hk, D, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    mk = lambda h: torch.randn((N, h, D), generator=g, device=DEV).to(torch.bfloat16)
    return mk(hq), mk(hk), mk(hk), mk(hq)


def _fwd_bwd(q, k, v, do, cu=None, causal=1):
    N, hq, D = q.shape
    hk = k.shape[1]
    scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((hq, N), dtype=torch.float32, device=DEV)
    uly.attn_fwd(q, k, v, o, lse, scale, cu, causal=causal)
    ws = torch.empty(uly.attn_bwd_workspace_size(N, hq, hk, D, q.dtype), dtype=torch.uint8, device=DEV)
    grads = [torch.empty(t.shape, dtype=torch.float32, device=DEV) for t in (q, k, v)]
    uly.attn_bwd_ex(q, k, v, o, do, lse, *grads, scale, ws, cu, causal=causal)
    torch.cuda.synchronize()
    return o, lse, grads


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("N,i0", [(4096, 2047), (3000, 1234), (777, 63)])
def test_causality_bitwise(N, i0):
    q, k, v, do = _inputs(N, 4, 1, 128, seed=N)
    o1, l1, g1 = _fwd_bwd(q, k, v, do)
    q2, k2, v2, do2 = (t.clone() for t in (q, k, v, do))
    for t in (q2, k2, v2, do2):
        t[i0 + 1:] = torch.randn(t[i0 + 1:].shape, device=DEV).to(t.dtype) * 3
    o2, l2, g2 = _fwd_bwd(q2, k2, v2, do2)
    r = slice(0, i0 + 1)
    assert _same(o1[r], o2[r]) and _same(l1[:, r], l2[:, r])
    assert _same(g1[0][r], g2[0][r])           # dQ of the rows up to i0
    assert not _same(o1[i0 + 1:], o2[i0 + 1:])  # the perturbation reached the later rows


@pytest.mark.parametrize("causal", [1, 0])
def test_document_isolation_bitwise(causal):
    lens = [700, 1, 0, 1300, 512, 1583]
    N = sum(lens)
    cu_host = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(cu_host).to(DEV)
    q, k, v, do = _inputs(N, 4, 1, 128, seed=7 + causal)
    o1, l1, g1 = _fwd_bwd(q, k, v, do, cu, causal)
    a, b = int(cu_host[3]), int(cu_host[4])     # the 1300-token document
    q2, k2, v2, do2 = (t.clone() for t in (q, k, v, do))
    for t in (q2, k2, v2, do2):
        t[a:b] = torch.randn(t[a:b].shape, device=DEV).to(t.dtype)
    o2, l2, g2 = _fwd_bwd(q2, k2, v2, do2, cu, causal)
    for r in (slice(0, a), slice(b, N)):
        assert _same(o1[r], o2[r]) and _same(l1[:, r], l2[:, r])
        for x, y in zip(g1, g2):
            assert _same(x[r], y[r])
    assert not _same(o1[a:b], o2[a:b])


@pytest.mark.parametrize("G", [4, 2, 8, 16])
def test_gqa_equals_repeated_kv(G):
    N, hk, D = 2048, 2, 128
    hq = hk * G
    q, k, v, do = _inputs(N, hq, hk, D, seed=11 * G)
    o1, l1, (dq1, dk1, dv1) = _fwd_bwd(q, k, v, do)
    kr = k.repeat_interleave(G, dim=1).contiguous()   # q head h reads kv head h // G
    vr = v.repeat_interleave(G, dim=1).contiguous()
    o2, l2, (dq2, dk2, dv2) = _fwd_bwd(q, kr, vr, do)
    assert _same(o1, o2) and _same(l1, l2)
    assert torch.allclose(dq1, dq2, atol=1e-5, rtol=1e-5)
    assert torch.allclose(dk1, dk2.view(N, hk, G, D).sum(dim=2), atol=1e-4, rtol=1e-4)
    assert torch.allclose(dv1, dv2.view(N, hk, G, D).sum(dim=2), atol=1e-4, rtol=1e-4)
