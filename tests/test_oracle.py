"""Pins for the CPU oracle: each check is independent of the oracle's own code.

The pages print no worked example, so the oracle is pinned by brute force on
tiny inputs (pure-Python loops), library routines (numpy slicing for the
redistributions, torch fp64 autograd and central finite differences for the
gradients), closed forms, and invariants the pages' statements imply:
  - the second all-to-all undoes the first ("Ulysses Sequence Parallelism
    ...", "All-to-All Communication" step) -> unpack(pack(x)) == x;
  - attention heads are independent ("Snowflake's Ulysses trick ...", second
    paragraph) -> a head group's result is the slice of all-heads attention;
  - tiled attention computes exact attention ("Ulysses Sequence Parallelism
    ...", quadratic-cost paragraph) -> the plain softmax definition.
Each test names the plausible oracle mistake it would catch.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (attn_ref, bf16_bits_to_f64, doc_tables, f32_bits_to_f64, merge_ref, pack_heads_ref, pack_qkv_ref,
                    pack_ref, replicated_kv_head, unpack_heads_ref, unpack_qkv_ref, unpack_ref)
from synthetic import cu_from_lengths


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- pack/unpack
def _shards(P, T, H, D, dtype=np.uint16, seed=0):
    r = _rng(seed)
    return [r.integers(0, np.iinfo(dtype).max, size=(T, H, D), dtype=dtype) for _ in range(P)]


@pytest.mark.parametrize("P,T,H,D,g", [(2, 3, 4, 2, 1), (4, 2, 8, 3, 2), (3, 5, 6, 1, 0), (1, 4, 3, 2, 0)])
def test_pack_matches_python_loops(P, T, H, D, g):
    """Brute force: nested loops over (shard, token, head, dim). Catches a
    swapped head/token index or a wrong group offset."""
    sh = _shards(P, T, H, D)
    hh = H // P
    want = np.zeros((P * T, hh, D), dtype=np.uint16)
    for j in range(P):
        for t in range(T):
            for h in range(hh):
                for d in range(D):
                    want[j * T + t, h, d] = sh[j][t, g * hh + h, d]
    assert np.array_equal(pack_ref(sh, g), want)


@pytest.mark.parametrize("P,T,H,D", [(4, 7, 8, 5), (8, 3, 32, 4), (2, 1, 2, 1)])
def test_pack_equals_concat_slice(P, T, H, D):
    """Closed form with library ops: concatenate shards along tokens, slice the
    group's heads. Catches non-contiguous shard order."""
    sh = _shards(P, T, H, D, dtype=np.uint32, seed=3)
    hh = H // P
    full = np.concatenate(sh, axis=0)
    for g in range(P):
        assert np.array_equal(pack_ref(sh, g), full[:, g * hh:(g + 1) * hh, :])


def test_unpack_inverts_pack_and_leaves_other_heads():
    """unpack(pack(X, g), g) rebuilds X from a copy whose g-slice was zeroed, and
    canary values in the other heads survive."""
    P, T, H, D = 4, 5, 8, 3
    sh = _shards(P, T, H, D, seed=5)
    hh = H // P
    for g in range(P):
        packed = pack_ref(sh, g)
        holed = [s.copy() for s in sh]
        for s in holed:
            s[:, g * hh:(g + 1) * hh, :] = 0
        back = unpack_ref(packed, holed, g)
        for a, b in zip(back, sh):
            assert np.array_equal(a, b)
        canary = [np.full_like(s, 0xBEEF) for s in sh]
        out = unpack_ref(packed, canary, g)
        for o, s in zip(out, sh):
            mask = np.ones(H, bool)
            mask[g * hh:(g + 1) * hh] = False
            assert np.all(o[:, mask, :] == 0xBEEF)
            assert np.array_equal(o[:, ~mask, :], s[:, ~mask, :])


def test_pack_all_groups_is_a_bijection():
    """Pack every group then unpack every group into zeros gives back X."""
    P, T, H, D = 4, 6, 12, 2
    sh = _shards(P, T, H, D, dtype=np.uint32, seed=9)
    cur = [np.zeros_like(s) for s in sh]
    for g in range(P):
        cur = unpack_ref(pack_ref(sh, g), cur, g)
    for a, b in zip(cur, sh):
        assert np.array_equal(a, b)


def test_pack_token_subset():
    P, T, H, D = 4, 9, 8, 3
    sh = _shards(P, T, H, D, seed=11)
    toks = np.array([0, 8, 9, 17, 35, 20])
    full = pack_ref(sh, 1)
    assert np.array_equal(pack_ref(sh, 1, tokens=toks), full[toks])
    base = [np.zeros_like(s) for s in sh]
    a = unpack_ref(full[toks], base, 1, tokens=toks)
    b = unpack_ref(full, base, 1)
    written = set()
    for n in toks:
        j, t = divmod(int(n), T)
        written.add((j, t))
        assert np.array_equal(a[j][t], b[j][t])
    for j in range(P):
        for t in range(T):
            if (j, t) not in written:
                assert not a[j][t].any()


# ------------------------------------------------------------- head-run pack/unpack
@pytest.mark.parametrize("P,T,H,D,h0,nh", [(2, 3, 4, 2, 1, 2), (4, 2, 2, 3, 1, 1), (1, 4, 5, 2, 0, 5), (3, 2, 6, 1, 5, 1)])
def test_pack_heads_matches_python_loops_and_slicing(P, T, H, D, h0, nh):
    """Brute force over (shard, token, head, dim), and numpy concatenate +
    slice. Catches an offset applied per group instead of per head."""
    sh = _shards(P, T, H, D, seed=51)
    want = np.zeros((P * T, nh, D), dtype=np.uint16)
    for j in range(P):
        for t in range(T):
            for h in range(nh):
                for d in range(D):
                    want[j * T + t, h, d] = sh[j][t, h0 + h, d]
    got = pack_heads_ref(sh, h0, nh)
    assert np.array_equal(got, want)
    assert np.array_equal(got, np.concatenate(sh, axis=0)[:, h0:h0 + nh])


def test_pack_heads_is_pack_for_a_group_and_inverts():
    P, T, H, D = 4, 5, 8, 3
    sh = _shards(P, T, H, D, seed=52)
    for g in range(P):
        packed = pack_heads_ref(sh, g * 2, 2)
        assert np.array_equal(packed, pack_ref(sh, g))
        canary = [np.full_like(s, 0xBEEF) for s in sh]
        for o, s in zip(unpack_heads_ref(packed, canary, g * 2, 2), sh):
            assert np.all(o[:, :g * 2] == 0xBEEF) and np.all(o[:, g * 2 + 2:] == 0xBEEF)
            assert np.array_equal(o[:, g * 2:g * 2 + 2], s[:, g * 2:g * 2 + 2])


def test_replicated_kv_head_attention_is_a_slice_of_all_heads():
    """Fewer kv heads than ranks (Hq = 8, Hkv = 2, P = 4): rank g's query
    heads with the one kv head it gathers give exactly the slice of
    attention over all heads (GQA with consecutive query heads per kv
    head). Catches a replicated head taken as g % Hkv instead of g*Hkv/P."""
    r = _rng(53)
    P, T, Hq, Hkv, D = 4, 3, 8, 2, 4
    N = P * T
    qs = [r.normal(size=(T, Hq, D)) for _ in range(P)]
    ks = [r.normal(size=(T, Hkv, D)) for _ in range(P)]
    vs = [r.normal(size=(T, Hkv, D)) for _ in range(P)]
    full = attn_ref(np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), 0.5, workers=1)
    assert [replicated_kv_head(g, P, Hq, Hkv) for g in range(P)] == [0, 0, 1, 1]
    for g in range(P):
        kv = replicated_kv_head(g, P, Hq, Hkv)
        q = pack_ref(qs, g)
        k, v = pack_heads_ref(ks, kv, 1), pack_heads_ref(vs, kv, 1)
        res = attn_ref(q, k, v, 0.5, workers=1)
        assert np.allclose(res["o"], full["o"][:, g * 2:(g + 1) * 2], atol=1e-13)


# ------------------------------------------------------- fused QKV pack/unpack
@pytest.mark.parametrize("P,T,Hq,Hkv,D,g", [(2, 3, 4, 2, 2, 1), (4, 2, 8, 4, 3, 3), (1, 4, 3, 1, 2, 0),
                                            (2, 2, 2, 2, 1, 0)])
def test_pack_qkv_matches_python_loops(P, T, Hq, Hkv, D, g):
    """Brute force over (shard, token, head, dim) with the section offsets
    written out. Catches a wrong section base (keys read from the query
    section, values from the keys) or a group offset scaled by the wrong head
    count."""
    H = Hq + 2 * Hkv
    sh = _shards(P, T, H, D, seed=21)
    hq, hk = Hq // P, Hkv // P
    want = [np.zeros((P * T, c, D), np.uint16) for c in (hq, hk, hk)]
    for j in range(P):
        for t in range(T):
            for d in range(D):
                for h in range(hq):
                    want[0][j * T + t, h, d] = sh[j][t, g * hq + h, d]
                for h in range(hk):
                    want[1][j * T + t, h, d] = sh[j][t, Hq + g * hk + h, d]
                    want[2][j * T + t, h, d] = sh[j][t, Hq + Hkv + g * hk + h, d]
    got = pack_qkv_ref(sh, Hq, Hkv, g)
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("P,T,Hq,Hkv,D", [(8, 3, 32, 8, 4), (4, 5, 4, 4, 2), (2, 1, 6, 2, 1)])
def test_pack_qkv_equals_split_and_slice(P, T, Hq, Hkv, D):
    """Closed form with library ops: split the fused heads into the query,
    key and value sections (numpy split), concatenate shards along tokens,
    slice each section's group heads."""
    sh = _shards(P, T, Hq + 2 * Hkv, D, dtype=np.uint32, seed=23)
    full = np.concatenate(sh, axis=0)
    qs, ks, vs = np.split(full, [Hq, Hq + Hkv], axis=1)
    hq, hk = Hq // P, Hkv // P
    for g in range(P):
        q, k, v = pack_qkv_ref(sh, Hq, Hkv, g)
        assert np.array_equal(q, qs[:, g * hq:(g + 1) * hq])
        assert np.array_equal(k, ks[:, g * hk:(g + 1) * hk])
        assert np.array_equal(v, vs[:, g * hk:(g + 1) * hk])


def test_unpack_qkv_inverts_pack_qkv_and_leaves_other_heads():
    """unpack_qkv(pack_qkv(X, g), g) rebuilds X from a copy whose group slices
    were zeroed; canaries in every other head survive; unpacking every group
    into zeros rebuilds X (the groups' slices tile the fused heads)."""
    P, T, Hq, Hkv, D = 4, 5, 8, 4, 3
    H = Hq + 2 * Hkv
    sh = _shards(P, T, H, D, seed=25)
    hq, hk = Hq // P, Hkv // P
    cur = [np.zeros_like(s) for s in sh]
    for g in range(P):
        packed = pack_qkv_ref(sh, Hq, Hkv, g)
        mine = np.zeros(H, bool)
        mine[g * hq:(g + 1) * hq] = True
        mine[Hq + g * hk:Hq + (g + 1) * hk] = True
        mine[Hq + Hkv + g * hk:Hq + Hkv + (g + 1) * hk] = True
        holed = [s.copy() for s in sh]
        for s in holed:
            s[:, mine, :] = 0
        for a, b in zip(unpack_qkv_ref(*packed, holed, Hq, Hkv, g), sh):
            assert np.array_equal(a, b)
        canary = [np.full_like(s, 0xBEEF) for s in sh]
        for o, s in zip(unpack_qkv_ref(*packed, canary, Hq, Hkv, g), sh):
            assert np.all(o[:, ~mine, :] == 0xBEEF)
            assert np.array_equal(o[:, mine, :], s[:, mine, :])
        cur = unpack_qkv_ref(*packed, cur, Hq, Hkv, g)
    for a, b in zip(cur, sh):
        assert np.array_equal(a, b)


def test_bits_decoding():
    """bf16 bits are the top half of fp32 (compared with torch's decoding)."""
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_bits_to_f64(bits), want)
    f = np.array([1.5, -2.25, 1e-30], dtype=np.float32)
    assert np.array_equal(f32_bits_to_f64(f.view(np.uint32)), f.astype(np.float64))


# ------------------------------------------------------------------- forward
def _doc_ids_loop(cu, N):
    ids = []
    for t in range(N):
        d = 0
        while not (cu[d] <= t < cu[d + 1]):
            d += 1
        ids.append(d)
    return ids


def brute_attn(q, k, v, scale, cu=None, causal=True):
    """Pure-Python loops, explicit softmax with math.exp."""
    N, hq, D = q.shape
    hk = k.shape[1]
    G = hq // hk
    cu = [0, N] if cu is None else list(cu)
    doc = _doc_ids_loop(cu, N)
    O = np.zeros((N, hq, D))
    L = np.zeros((hq, N))
    for h in range(hq):
        kh = h // G
        for i in range(N):
            js = [j for j in range(N) if doc[j] == doc[i] and (j <= i or not causal)]
            s = [scale * sum(q[i, h, d] * k[j, kh, d] for d in range(D)) for j in js]
            mx = max(s)
            z = sum(math.exp(x - mx) for x in s)
            lse = mx + math.log(z)
            for x, j in zip(s, js):
                p = math.exp(x - lse)
                for d in range(D):
                    O[i, h, d] += p * v[j, kh, d]
            L[h, i] = lse
    return O, L


@pytest.mark.parametrize("N,hq,hk,D,lens", [
    (9, 2, 1, 3, None), (12, 4, 2, 2, [5, 0, 4, 3]), (7, 1, 1, 4, [1, 6]), (16, 4, 1, 2, [3, 3, 0, 10]),
])
def test_fwd_matches_python_loops(N, hq, hk, D, lens):
    r = _rng(N)
    q, k, v = r.normal(size=(N, hq, D)), r.normal(size=(N, hk, D)), r.normal(size=(N, hk, D))
    cu = None if lens is None else cu_from_lengths(lens)
    O, L = brute_attn(q, k, v, 0.7, cu)
    res = attn_ref(q, k, v, 0.7, cu, workers=1)
    assert np.allclose(res["o"], O, rtol=0, atol=1e-12)
    assert np.allclose(res["lse"], L, rtol=0, atol=1e-12)


def test_fwd_noncausal_matches_python_loops():
    r = _rng(2)
    q, k, v = r.normal(size=(8, 2, 3)), r.normal(size=(8, 1, 3)), r.normal(size=(8, 1, 3))
    cu = cu_from_lengths([3, 5])
    O, L = brute_attn(q, k, v, 0.5, cu, causal=False)
    res = attn_ref(q, k, v, 0.5, cu, causal=False, workers=1)
    assert np.allclose(res["o"], O, atol=1e-12) and np.allclose(res["lse"], L, atol=1e-12)


def test_fwd_hand_computed():
    """Worked by hand: D=1, scale=1, q=1, keys 0, ln2, ln3 -> row 2 weights
    (1,2,3)/6, LSE = ln 6; row 1 weights (1,2)/3, LSE = ln 3; row 0 LSE 0."""
    q = np.ones((3, 1, 1))
    k = np.array([0.0, math.log(2), math.log(3)]).reshape(3, 1, 1)
    v = np.array([6.0, 12.0, 18.0]).reshape(3, 1, 1)
    res = attn_ref(q, k, v, 1.0, workers=1)
    assert np.allclose(res["lse"][0], [0.0, math.log(3), math.log(6)], atol=1e-14)
    # row 1: (6 + 2*12)/3 = 10 ; row 2: (6 + 24 + 54)/6 = 14
    assert np.allclose(res["o"][:, 0, 0], [6.0, 10.0, 14.0], atol=1e-12)


def test_softmax_rows_sum_to_one():
    """With V = 1 every output is sum_j P_ij = 1 (catches a missing normaliser
    or a mask that drops the diagonal from the denominator only)."""
    r = _rng(4)
    N = 300
    q, k = r.normal(size=(N, 4, 8)) * 3, r.normal(size=(N, 1, 8)) * 3
    v = np.ones((N, 1, 8))
    res = attn_ref(q, k, v, 0.35, cu_from_lengths([100, 1, 50, 149]), workers=2)
    assert np.allclose(res["o"], 1.0, atol=1e-13)


def test_causality():
    """Perturbing tokens > i leaves rows <= i unchanged (catches j < i vs
    j <= i slips in the other direction and a missing causal mask)."""
    r = _rng(5)
    N, i = 64, 37
    q, k, v = r.normal(size=(N, 2, 4)), r.normal(size=(N, 1, 4)), r.normal(size=(N, 1, 4))
    a = attn_ref(q, k, v, 0.5, workers=1)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[i + 1:] += 5
    v2[i + 1:] -= 3
    q2[i + 1:] *= -2
    b = attn_ref(q2, k2, v2, 0.5, workers=1)
    assert np.array_equal(a["o"][:i + 1], b["o"][:i + 1])
    assert np.array_equal(a["lse"][:, :i + 1], b["lse"][:, :i + 1])
    # and the diagonal is attended: changing v_i changes o_i
    v3 = v.copy()
    v3[i] += 1
    c = attn_ref(q, k, v3, 0.5, workers=1)
    assert not np.allclose(a["o"][i], c["o"][i])


def test_q_zero_closed_form():
    """Q = 0: uniform weights over [doc_start(i), i] -> O_i = prefix mean of V in
    the document, LSE_i = log(i - doc_start + 1)."""
    r = _rng(6)
    lens = [5, 0, 17, 1, 41]
    N = sum(lens)
    cu = cu_from_lengths(lens)
    q = np.zeros((N, 2, 3))
    k, v = r.normal(size=(N, 2, 3)), r.normal(size=(N, 2, 3))
    res = attn_ref(q, k, v, 1.3, cu, workers=1)
    for i in range(N):
        s = max(int(c) for c in cu if c <= i)
        assert np.allclose(res["o"][i], v[s:i + 1].mean(axis=0), atol=1e-13)
        assert np.allclose(res["lse"][:, i], math.log(i - s + 1), atol=1e-13)


def test_single_token_document():
    r = _rng(7)
    cu = cu_from_lengths([4, 1, 3])
    q, k, v = r.normal(size=(8, 2, 5)), r.normal(size=(8, 1, 5)), r.normal(size=(8, 1, 5))
    res = attn_ref(q, k, v, 0.4, cu, workers=1)
    assert np.allclose(res["o"][4], v[4, [0, 0]], atol=1e-14)
    assert np.allclose(res["lse"][:, 4], 0.4 * (q[4] @ k[4, 0]), atol=1e-14)


def test_head_group_is_slice_of_all_heads():
    """Heads are independent: group g's result equals the g-slice of attention
    over all heads with the global GQA map (kv head = h // (Hq/Hkv))."""
    r = _rng(8)
    N, Hq, Hkv, D, P = 40, 16, 4, 3, 4
    q, k, v = r.normal(size=(N, Hq, D)), r.normal(size=(N, Hkv, D)), r.normal(size=(N, Hkv, D))
    do = r.normal(size=(N, Hq, D))
    full = attn_ref(q, k, v, 0.6, do=do, workers=1)
    hq, hk = Hq // P, Hkv // P
    for g in range(P):
        sl = attn_ref(q[:, g * hq:(g + 1) * hq], k[:, g * hk:(g + 1) * hk], v[:, g * hk:(g + 1) * hk], 0.6,
                      do=do[:, g * hq:(g + 1) * hq], workers=1)
        assert np.allclose(sl["o"], full["o"][:, g * hq:(g + 1) * hq], atol=1e-13)
        assert np.allclose(sl["dk"], full["dk"][:, g * hk:(g + 1) * hk], atol=1e-12)
        assert np.allclose(sl["dq"], full["dq"][:, g * hq:(g + 1) * hq], atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    """GQA forward equals MHA on K/V repeated per q head; GQA dK/dV equal the
    per-q-head MHA gradients summed over each kv head's q heads."""
    r = _rng(9)
    N, hq, hk, D = 33, 4, 1, 6
    q, k, v, do = (r.normal(size=s) for s in [(N, hq, D), (N, hk, D), (N, hk, D), (N, hq, D)])
    cu = cu_from_lengths([10, 23])
    g = attn_ref(q, k, v, 0.3, cu, do=do, workers=1)
    m = attn_ref(q, np.repeat(k, hq // hk, axis=1), np.repeat(v, hq // hk, axis=1), 0.3, cu, do=do, workers=1)
    assert np.allclose(g["o"], m["o"], atol=1e-13)
    assert np.allclose(g["dq"], m["dq"], atol=1e-12)
    assert np.allclose(g["dk"][:, 0], m["dk"].sum(axis=1), atol=1e-12)
    assert np.allclose(g["dv"][:, 0], m["dv"].sum(axis=1), atol=1e-12)


def test_varlen_equals_separate_documents():
    r = _rng(10)
    lens = [7, 0, 12, 1, 20]
    N = sum(lens)
    cu = cu_from_lengths(lens)
    q, k, v, do = (r.normal(size=s) for s in [(N, 2, 4), (N, 1, 4), (N, 1, 4), (N, 2, 4)])
    whole = attn_ref(q, k, v, 0.5, cu, do=do, workers=1)
    for a, b in zip(cu[:-1], cu[1:]):
        if a == b:
            continue
        part = attn_ref(q[a:b], k[a:b], v[a:b], 0.5, do=do[a:b], workers=1)
        assert np.allclose(whole["o"][a:b], part["o"], atol=1e-13)
        assert np.allclose(whole["lse"][:, a:b], part["lse"], atol=1e-13)
        for key in ("dq", "dk", "dv"):
            assert np.allclose(whole[key][a:b], part[key], atol=1e-12)


def test_prefix_and_row_subsets():
    """Rows < M depend only on tokens < M; evaluating a row subset gives the
    same rows as the full run; a tail of rows gives exact dK/dV for the tail's
    key columns."""
    r = _rng(11)
    N, M = 200, 77
    cu = cu_from_lengths([50, 90, 60])
    q, k, v, do = (r.normal(size=s) for s in [(N, 4, 4), (N, 1, 4), (N, 1, 4), (N, 4, 4)])
    full = attn_ref(q, k, v, 0.5, cu, do=do, workers=3)
    pre = attn_ref(q[:M], k[:M], v[:M], 0.5, cu_from_lengths([50, 27]), do=do[:M], workers=1)
    assert np.allclose(pre["o"], full["o"][:M], atol=1e-13)
    rows = np.array([0, 1, 49, 50, 51, 139, 140, 199])
    sub = attn_ref(q, k, v, 0.5, cu, do=do, rows=rows, workers=2)
    assert np.allclose(sub["o"], full["o"][rows], atol=1e-13)
    assert np.allclose(sub["lse"], full["lse"][:, rows], atol=1e-13)
    assert np.allclose(sub["dq"], full["dq"][rows], atol=1e-12)
    tail = attn_ref(q, k, v, 0.5, cu, do=do, rows=np.arange(120, N), workers=2)
    assert np.allclose(tail["dk"][120:], full["dk"][120:], atol=1e-12)
    assert np.allclose(tail["dv"][120:], full["dv"][120:], atol=1e-12)


# ------------------------------------------------------------------ backward
def _loss(q, k, v, do, scale, cu):
    return float((attn_ref(q, k, v, scale, cu, workers=1)["o"] * do).sum())


def test_backward_finite_differences():
    """Central differences of L = sum(dO * O) in fp64 (catches a wrong sign, a
    missing scale, a dropped delta term, a transposed product)."""
    r = _rng(12)
    N, hq, hk, D = 7, 2, 1, 3
    cu = cu_from_lengths([3, 4])
    q, k, v, do = (r.normal(size=s) for s in [(N, hq, D), (N, hk, D), (N, hk, D), (N, hq, D)])
    res = attn_ref(q, k, v, 0.8, cu, do=do, workers=1)
    h = 1e-6
    for name, x, grad in (("q", q, res["dq"]), ("k", k, res["dk"]), ("v", v, res["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, 0.8, cu)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, 0.8, cu)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err < 1e-6, (name, err)


def test_backward_matches_torch_autograd():
    """torch fp64 autograd through an explicit masked softmax on the CPU."""
    r = _rng(13)
    N, hq, hk, D = 29, 4, 2, 5
    lens = [9, 0, 11, 9]
    cu = cu_from_lengths(lens)
    q, k, v, do = (r.normal(size=s) for s in [(N, hq, D), (N, hk, D), (N, hk, D), (N, hq, D)])
    res = attn_ref(q, k, v, 0.45, cu, do=do, workers=1)
    doc = torch.tensor(np.repeat(np.arange(len(lens)), lens))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    idx = torch.arange(N)
    mask = (idx[None, :] <= idx[:, None]) & (doc[None, :] == doc[:, None])
    outs = []
    for h in range(hq):
        s = 0.45 * tq[:, h] @ tk[:, h // (hq // hk)].T
        s = s.masked_fill(~mask, float("-inf"))
        outs.append(torch.softmax(s, dim=1) @ tv[:, h // (hq // hk)])
    o = torch.stack(outs, dim=1)
    (o * torch.tensor(do)).sum().backward()
    assert np.allclose(res["o"], o.detach().numpy(), atol=1e-13)
    assert np.allclose(res["dq"], tq.grad.numpy(), atol=1e-12)
    assert np.allclose(res["dk"], tk.grad.numpy(), atol=1e-12)
    assert np.allclose(res["dv"], tv.grad.numpy(), atol=1e-12)


def test_backward_document_sum_invariants():
    """Softmax is shift invariant in k, so sum_{j in doc} dK_j = 0; each P row
    sums to 1, so sum_{j in doc} dV_j = sum_h sum_{i in doc} dO_{h,i}."""
    r = _rng(14)
    lens = [40, 1, 0, 87]
    N = sum(lens)
    cu = cu_from_lengths(lens)
    q, k, v, do = (r.normal(size=s) for s in [(N, 4, 8), (N, 1, 8), (N, 1, 8), (N, 4, 8)])
    res = attn_ref(q, k, v, 0.35, cu, do=do, workers=2)
    for a, b in zip(cu[:-1], cu[1:]):
        if a == b:
            continue
        assert np.allclose(res["dk"][a:b].sum(axis=0), 0, atol=1e-11)
        assert np.allclose(res["dv"][a:b].sum(axis=0)[0], do[a:b].sum(axis=(0, 1)), atol=1e-11)


def test_backward_q_zero_closed_form():
    """Q = 0: P_ij = 1/(i - s + 1) on the document prefix, so
    dV_j = sum_h sum_{i in doc, i >= j} dO_{h,i} / (i - s + 1)."""
    r = _rng(15)
    lens = [6, 10]
    N = sum(lens)
    cu = cu_from_lengths(lens)
    q = np.zeros((N, 2, 3))
    k, v, do = r.normal(size=(N, 1, 3)), r.normal(size=(N, 1, 3)), r.normal(size=(N, 2, 3))
    res = attn_ref(q, k, v, 0.9, cu, do=do, workers=1)
    for j in range(N):
        s = 0 if j < 6 else 6
        e = 6 if j < 6 else N
        want = sum(do[i].sum(axis=0) / (i - s + 1) for i in range(j, e))
        assert np.allclose(res["dv"][j, 0], want, atol=1e-13)


# ------------------------------------------- attention with document-only masks
def test_noncausal_backward_finite_differences():
    """Document-only mask (every token of a document sees the whole document):
    central differences of L = sum(dO * O), with O from the pure-Python loops,
    against the oracle's analytic gradients (catches a causal bound left in the
    backward, or a key-side bound taken from the query's document)."""
    r = _rng(31)
    N, hq, hk, D = 7, 2, 1, 3
    cu = cu_from_lengths([4, 3])
    q, k, v, do = (r.normal(size=s) for s in [(N, hq, D), (N, hk, D), (N, hk, D), (N, hq, D)])
    res = attn_ref(q, k, v, 0.7, cu, do=do, causal=False, workers=1)
    h = 1e-6

    def loss(args):
        O, _ = brute_attn(args["q"], args["k"], args["v"], 0.7, cu, causal=False)
        return float((O * do).sum())
    for name, x, grad in (("q", q, res["dq"]), ("k", k, res["dk"]), ("v", v, res["dv"])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args)
            args[name] = xm
            lm = loss(args)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - grad).max() / max(np.abs(grad).max(), 1e-30)
        assert err < 1e-6, (name, err)


def test_noncausal_q_zero_closed_form():
    """Q = 0 with a document-only mask: every row of a document of length L
    averages all its values, LSE = log L, and dV_j = sum_h sum_{i in doc}
    dO_{h,i} / L."""
    r = _rng(32)
    lens = [5, 1, 0, 9]
    N = sum(lens)
    cu = cu_from_lengths(lens)
    q = np.zeros((N, 2, 4))
    k, v, do = r.normal(size=(N, 1, 4)), r.normal(size=(N, 1, 4)), r.normal(size=(N, 2, 4))
    res = attn_ref(q, k, v, 0.6, cu, do=do, causal=False, workers=1)
    for a, b in zip(cu[:-1], cu[1:]):
        if a == b:
            continue
        L = b - a
        mean_v = v[a:b, 0].mean(axis=0)
        for i in range(a, b):
            for h in range(2):
                assert np.allclose(res["o"][i, h], mean_v, atol=1e-13)
                assert abs(res["lse"][h, i] - math.log(L)) < 1e-13
        want_dv = do[a:b].sum(axis=(0, 1)) / L
        for j in range(a, b):
            assert np.allclose(res["dv"][j, 0], want_dv, atol=1e-13)


def test_noncausal_matches_torch_autograd():
    """torch fp64 autograd through an explicit document-masked softmax."""
    r = _rng(33)
    lens = [7, 0, 12, 4]
    N, hq, hk, D = sum(lens), 4, 2, 5
    cu = cu_from_lengths(lens)
    q, k, v, do = (r.normal(size=s) for s in [(N, hq, D), (N, hk, D), (N, hk, D), (N, hq, D)])
    res = attn_ref(q, k, v, 0.5, cu, do=do, causal=False, workers=1)
    doc = torch.tensor(np.repeat(np.arange(len(lens)), lens))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = doc[None, :] == doc[:, None]
    outs = []
    for h in range(hq):
        sc = 0.5 * tq[:, h] @ tk[:, h // (hq // hk)].T
        outs.append(torch.softmax(sc.masked_fill(~mask, float("-inf")), dim=1) @ tv[:, h // (hq // hk)])
    o = torch.stack(outs, dim=1)
    (o * torch.tensor(do)).sum().backward()
    assert np.allclose(res["o"], o.detach().numpy(), atol=1e-13)
    assert np.allclose(res["dq"], tq.grad.numpy(), atol=1e-12)
    assert np.allclose(res["dk"], tk.grad.numpy(), atol=1e-12)
    assert np.allclose(res["dv"], tv.grad.numpy(), atol=1e-12)


# ------------------------------------------------------------ LSE merge of key chunks
def test_merge_of_key_chunks_equals_full_attention():
    """Causal attention over N = 4 chunks of T tokens, computed chunk pair by
    chunk pair (query chunk i against key chunk c: no mask for c < i, causal
    within the chunk for c = i) and merged, equals attention over the whole
    sequence (the identity ring-style attention rests on)."""
    r = _rng(41)
    P, T, hq, hk, D = 4, 9, 4, 2, 5
    N = P * T
    q, k, v = r.normal(size=(N, hq, D)), r.normal(size=(N, hk, D)), r.normal(size=(N, hk, D))
    full = attn_ref(q, k, v, 0.6, workers=1)
    for i in range(P):
        qi = slice(i * T, (i + 1) * T)
        parts = []
        for c in range(i + 1):
            kc = slice(c * T, (c + 1) * T)
            parts.append(attn_ref(q[qi], k[kc], v[kc], 0.6, causal=(c == i), workers=1))
        o, lse = merge_ref([p["o"] for p in parts], [p["lse"] for p in parts])
        assert np.allclose(o, full["o"][qi], atol=1e-12)
        assert np.allclose(lse, full["lse"][:, qi], atol=1e-12)


def test_merge_brute_force_and_edge_cases():
    """Explicit loops with math.exp/log; one part is the identity; parts
    commute; a part with lse = -inf adds nothing; all parts -inf -> o = 0,
    lse = -inf."""
    r = _rng(42)
    N, hq, D, C = 5, 2, 3, 3
    o_parts = [r.normal(size=(N, hq, D)) for _ in range(C)]
    lse_parts = [r.normal(size=(hq, N)) * 3 for _ in range(C)]
    o, lse = merge_ref(o_parts, lse_parts)
    for h in range(hq):
        for i in range(N):
            z = sum(math.exp(lse_parts[c][h, i]) for c in range(C))
            assert abs(lse[h, i] - math.log(z)) < 1e-12
            for d in range(D):
                want = sum(math.exp(lse_parts[c][h, i]) / z * o_parts[c][i, h, d] for c in range(C))
                assert abs(o[i, h, d] - want) < 1e-12
    o1, l1 = merge_ref(o_parts[:1], lse_parts[:1])
    assert np.allclose(o1, o_parts[0], atol=1e-15) and np.allclose(l1, lse_parts[0], atol=1e-15)
    o2, l2 = merge_ref(o_parts[::-1], lse_parts[::-1])
    assert np.allclose(o2, o, atol=1e-13) and np.allclose(l2, lse, atol=1e-13)
    dead = np.full((hq, N), -np.inf)
    o3, l3 = merge_ref(o_parts + [r.normal(size=(N, hq, D))], lse_parts + [dead])
    assert np.allclose(o3, o, atol=1e-13) and np.allclose(l3, lse, atol=1e-13)
    o4, l4 = merge_ref(o_parts[:2], [dead, dead])
    assert np.all(o4 == 0) and np.all(l4 == -np.inf)


def test_doc_tables_and_errors():
    doc, start = doc_tables(np.array([0, 3, 3, 5]), 5)
    assert list(doc) == [0, 0, 0, 2, 2]
    assert list(start) == [0, 0, 0, 3, 3]
    with pytest.raises(ValueError):
        doc_tables(np.array([0, 4, 3, 5]), 5)
    with pytest.raises(ValueError):
        doc_tables(np.array([1, 5]), 5)
