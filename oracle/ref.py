"""Plain, slow fp64 reference for the Ulysses one-GPU hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring). No blocking, fusion or
reordering beyond what the definitions state: query rows are processed in
blocks only to bound memory, and each block builds its full masked score
matrix over every key that the mask can admit.

Notation (pages: "Ulysses Sequence Parallelism: Training with Million-Token
Contexts" and "Snowflake's Ulysses trick trains transformers on million-token
contexts across GPUs"):
  P ranks; rank j holds the contiguous token block [j*T, (j+1)*T) of the
  N = P*T tokens (the "Sequence Sharding" step; the token-range symbols were
  lost from the page, contiguous blocks are the plain reading).
  H heads in a shard; head group g owns heads [g*hh, (g+1)*hh), hh = H/P
  (each GPU keeps "a subset of attention heads"; contiguous is the plain
  reading).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np


# ---------------------------------------------------------------------------
# value decoding (the oracle's own; the GPU path has its own conversions)
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: bf16 is the top half of an IEEE fp32."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits).astype(np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# the two redistributions, as explicit integer index arithmetic on raw bits
# ---------------------------------------------------------------------------
def _check_shards(shards):
    P = len(shards)
    if P < 1:
        raise ValueError("need at least one shard")
    T, H, D = shards[0].shape
    for s in shards:
        if s.shape != (T, H, D) or s.dtype != shards[0].dtype:
            raise ValueError("shards must share shape and dtype")
    if H % P:
        raise ValueError("head count must be divisible by the number of shards")
    return P, T, H, D


def pack_ref(shards, group: int, tokens=None) -> np.ndarray:
    """Sequence-sharded -> head-sharded, for head group `group`.

    The first all-to-all leaves each GPU with every token of the sequence for
    its own subset of heads ("Snowflake's Ulysses trick ...", second
    paragraph). Output row n (global token n = j*T + t) holds heads
    [group*hh, (group+1)*hh) of token t of shard j:

        out[n, h, d] = shard_j[t, group*hh + h, d],  j = n // T, t = n % T.

    shards: P arrays [T, H, D] of raw bits (any integer dtype; copied, never
    interpreted). tokens: optional array of global token indices; if given,
    only those output rows are produced, in that order. Returns [len, hh, D].
    """
    P, T, H, D = _check_shards(shards)
    hh = H // P
    if not 0 <= group < P:
        raise ValueError("group out of range")
    N = P * T
    n_rows = N if tokens is None else len(tokens)
    tok = np.arange(N, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    # flat output index -> (token, head, dim)
    o = np.arange(n_rows * hh * D, dtype=np.int64)
    d = o % D
    h = (o // D) % hh
    r = o // (hh * D)
    n = tok[r]
    j = n // T
    t = n % T
    src = (t * H + group * hh + h) * D + d  # flat index inside shard j
    out = np.empty(n_rows * hh * D, dtype=shards[0].dtype)
    flats = [s.reshape(-1) for s in shards]
    for jj in range(P):
        sel = j == jj
        out[sel] = flats[jj][src[sel]]
    return out.reshape(n_rows, hh, D)


def unpack_ref(packed: np.ndarray, shards, group: int, tokens=None):
    """Head-sharded -> sequence-sharded: the inverse redistribution ("Ulysses
    Sequence Parallelism ...", the "All-to-All Communication" step).

        shard_j[t, group*hh + h, d] = packed[j*T + t, h, d]

    for every j, t, h, d; heads outside the group are left as they are.
    `shards` supplies the prior contents and is not modified: new arrays are
    returned. With `tokens`, `packed` holds only those rows (in that order) and
    only they are written.
    """
    P, T, H, D = _check_shards(shards)
    hh = H // P
    if not 0 <= group < P:
        raise ValueError("group out of range")
    N = P * T
    tok = np.arange(N, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    if packed.shape != (len(tok), hh, D):
        raise ValueError("packed shape mismatch")
    out = [s.copy().reshape(-1) for s in shards]
    o = np.arange(len(tok) * hh * D, dtype=np.int64)
    d = o % D
    h = (o // D) % hh
    r = o // (hh * D)
    n = tok[r]
    j = n // T
    t = n % T
    dst = (t * H + group * hh + h) * D + d
    flat_in = packed.reshape(-1)
    for jj in range(P):
        sel = j == jj
        out[jj][dst[sel]] = flat_in[o[sel]]
    return [x.reshape(T, H, D) for x in out]


def pack_heads_ref(shards, head0: int, nheads: int) -> np.ndarray:
    """The redistribution for any run of heads [head0, head0 + nheads):

        out[n, h, d] = shard_j[t, head0 + h, d],  n = j*T + t.

    With head0 = group*H/P and nheads = H/P this is pack_ref. With fewer
    key/value heads than ranks the pages say nothing; the reading taken is
    that kv heads are replicated and rank g gathers the one its query heads
    use (replicated_kv_head)."""
    P, T, H, D = _check_shards_any(shards)
    if not (nheads >= 1 and 0 <= head0 <= H - nheads):
        raise ValueError("head run out of range")
    o = np.arange(P * T * nheads * D, dtype=np.int64)
    d = o % D
    h = (o // D) % nheads
    n = o // (nheads * D)
    j, t = n // T, n % T
    src = (t * H + head0 + h) * D + d
    out = np.empty(o.size, dtype=shards[0].dtype)
    flats = [s.reshape(-1) for s in shards]
    for jj in range(P):
        sel = j == jj
        out[sel] = flats[jj][src[sel]]
    return out.reshape(P * T, nheads, D)


def unpack_heads_ref(packed: np.ndarray, shards, head0: int, nheads: int):
    """Inverse of pack_heads_ref: shard_j[t, head0 + h, d] = packed[j*T + t,
    h, d]; other heads keep the values in `shards` (new arrays returned)."""
    P, T, H, D = _check_shards_any(shards)
    if packed.shape != (P * T, nheads, D) or not (nheads >= 1 and 0 <= head0 <= H - nheads):
        raise ValueError("shape or head run mismatch")
    out = [s.copy().reshape(-1) for s in shards]
    o = np.arange(P * T * nheads * D, dtype=np.int64)
    d = o % D
    h = (o // D) % nheads
    n = o // (nheads * D)
    j, t = n // T, n % T
    dst = (t * H + head0 + h) * D + d
    flat_in = packed.reshape(-1)
    for jj in range(P):
        sel = j == jj
        out[jj][dst[sel]] = flat_in[o[sel]]
    return [x.reshape(T, H, D) for x in out]


def replicated_kv_head(g: int, P: int, Hq: int, Hkv: int) -> int:
    """The kv head rank g needs when Hkv < P: its query heads
    [g*Hq/P, (g+1)*Hq/P) all read kv head floor(h / (Hq/Hkv)) (consecutive
    query heads share a kv head), which is floor(g * Hkv / P) when P is a
    multiple of Hkv."""
    if Hq % P or P % Hkv or Hq % Hkv:
        raise ValueError("needs P | Hq, Hkv | P and Hkv | Hq")
    heads = {h // (Hq // Hkv) for h in range(g * (Hq // P), (g + 1) * (Hq // P))}
    assert len(heads) == 1
    return heads.pop()


def _check_shards_any(shards):
    P = len(shards)
    if P < 1:
        raise ValueError("need at least one shard")
    T, H, D = shards[0].shape
    for s in shards:
        if s.shape != (T, H, D) or s.dtype != shards[0].dtype:
            raise ValueError("shards must share shape and dtype")
    return P, T, H, D


def _qkv_sections(shards, Hq: int, Hkv: int, group: int):
    P = len(shards)
    if P < 1:
        raise ValueError("need at least one shard")
    T, H, D = shards[0].shape
    for s in shards:
        if s.shape != (T, H, D) or s.dtype != shards[0].dtype:
            raise ValueError("shards must share shape and dtype")
    if H != Hq + 2 * Hkv or Hq % P or Hkv % P:
        raise ValueError("fused shards need Hq + 2*Hkv heads with Hq, Hkv divisible by P")
    if not 0 <= group < P:
        raise ValueError("group out of range")
    hq, hk = Hq // P, Hkv // P
    # (first head of the group's slice inside a shard token, heads in the slice)
    return P, T, H, D, [(group * hq, hq), (Hq + group * hk, hk), (Hq + Hkv + group * hk, hk)]


def pack_qkv_ref(shards, Hq: int, Hkv: int, group: int):
    """The first redistribution applied to a fused QKV projection output (the
    all-to-all follows each GPU's local QKV projections: "Snowflake's Ulysses
    trick ...", second paragraph). Layout reading: a shard token holds the Hq
    query heads, then the Hkv key heads, then the Hkv value heads. For the
    section starting at head b with the group's slice of c heads:

        out[n, h, d] = shard_j[t, b + h, d],  n = j*T + t, h < c,

    with b = group*hq (queries), Hq + group*hk (keys), Hq + Hkv + group*hk
    (values). shards: P arrays [T, Hq + 2*Hkv, D] of raw bits. Returns the
    three packed arrays (q [N, hq, D], k and v [N, hk, D]).
    """
    P, T, H, D, sections = _qkv_sections(shards, Hq, Hkv, group)
    flats = [s.reshape(-1) for s in shards]
    outs = []
    for b, c in sections:
        o = np.arange(P * T * c * D, dtype=np.int64)
        d = o % D
        h = (o // D) % c
        n = o // (c * D)
        j, t = n // T, n % T
        src = (t * H + b + h) * D + d
        out = np.empty(o.size, dtype=shards[0].dtype)
        for jj in range(P):
            sel = j == jj
            out[sel] = flats[jj][src[sel]]
        outs.append(out.reshape(P * T, c, D))
    return tuple(outs)


def unpack_qkv_ref(dq: np.ndarray, dk: np.ndarray, dv: np.ndarray, shards, Hq: int, Hkv: int, group: int):
    """Inverse of pack_qkv_ref (the backward's mirror of the second
    redistribution): shard_j[t, b + h, d] = packed[j*T + t, h, d] for the
    three sections; heads outside the group's slices keep the values in
    `shards`, which is not modified (new arrays are returned)."""
    P, T, H, D, sections = _qkv_sections(shards, Hq, Hkv, group)
    out = [s.copy().reshape(-1) for s in shards]
    for packed, (b, c) in zip((dq, dk, dv), sections):
        if packed.shape != (P * T, c, D):
            raise ValueError("packed shape mismatch")
        o = np.arange(P * T * c * D, dtype=np.int64)
        d = o % D
        h = (o // D) % c
        n = o // (c * D)
        j, t = n // T, n % T
        dst = (t * H + b + h) * D + d
        flat_in = packed.reshape(-1)
        for jj in range(P):
            sel = j == jj
            out[jj][dst[sel]] = flat_in[o[sel]]
    return [x.reshape(T, H, D) for x in out]


# ---------------------------------------------------------------------------
# documents
# ---------------------------------------------------------------------------
def doc_tables(cu_seqlens, N: int):
    """Per-token document id and document start.

    cu_seqlens: non-decreasing offsets, first 0, last N (None -> one document
    of N tokens). Empty documents (repeated offsets) own no tokens."""
    if cu_seqlens is None:
        cu = np.array([0, N], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != N or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing from 0 to N")
    tok = np.arange(N, dtype=np.int64)
    doc = np.searchsorted(cu, tok, side="right") - 1
    start = cu[doc]
    return doc, start


# ---------------------------------------------------------------------------
# attention: exact masked softmax and its analytic gradients
# ---------------------------------------------------------------------------
def _block(h, rows, q, k, v, do, scale, G, doc, start, causal):
    """One head h, one block of query rows: the plain definition.

    Scores S_ij = scale * q_i . k_j over keys j that the mask can admit; the
    mask keeps j <= i (causal) and doc(j) == doc(i). LSE_i = log sum_j
    exp(S_ij); P_ij = exp(S_ij - LSE_i); O_i = sum_j P_ij v_j.

    With upstream gradient dO (loss L = sum dO * O):
      delta_i = sum_d dO_id O_id
      dV_j   += sum_i P_ij dO_i
      dP_ij   = dO_i . v_j
      dS_ij   = P_ij (dP_ij - delta_i)
      dQ_i    = scale * sum_j dS_ij k_j
      dK_j   += scale * sum_i dS_ij q_i
    """
    kvh = h // G
    N = q.shape[0]
    # keys outside [lo, hi) are masked for every row of the block
    lo = int(start[rows].min())
    hi = int(rows.max()) + 1 if causal else N
    if not causal:
        # the last token of the last document any row belongs to
        last_doc = doc[rows].max()
        hi = int(np.searchsorted(doc, last_doc, side="right"))
    keys = np.arange(lo, hi, dtype=np.int64)
    qi = q[rows, h, :]                      # [B, D]
    kj = k[lo:hi, kvh, :]                   # [W, D]
    vj = v[lo:hi, kvh, :]
    S = scale * (qi @ kj.T)                 # [B, W]
    allowed = doc[keys][None, :] == doc[rows][:, None]
    if causal:
        allowed &= keys[None, :] <= rows[:, None]
    S = np.where(allowed, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]
    Pm = np.exp(S - lse[:, None])
    O = Pm @ vj
    res = {"o": O, "lse": lse}
    if do is not None:
        doi = do[rows, h, :]
        delta = (doi * O).sum(axis=1)
        dV = Pm.T @ doi
        dP = doi @ vj.T
        dS = Pm * (dP - delta[:, None])
        res["delta"] = delta
        res["dq"] = scale * (dS @ kj)
        res["dk"] = scale * (dS.T @ qi)
        res["dv"] = dV
        res["lo"], res["hi"] = lo, hi
    return res


def attn_ref(q, k, v, scale: float, cu_seqlens=None, do=None, rows=None,
             causal: bool = True, workers: int | None = None,
             max_block_elems: int = 1 << 23):
    """Exact attention for one head group, fp64.

    q: [N, hq, D]; k, v: [N, hk, D] (real arrays; converted to fp64);
    local q head h reads kv head h // (hq // hk) (consecutive q heads share a
    kv head). do: optional upstream gradient [N, hq, D].
    rows: optional sorted query rows to evaluate (default: all N).

    Returns a dict with 'rows', 'o' [R, hq, D], 'lse' [hq, R] (natural log),
    and with `do`: 'delta' [hq, R], 'dq' [R, hq, D], and 'dk', 'dv' [N, hk, D]
    holding the contributions of the evaluated rows only (complete for every
    key column j when the evaluated rows include all rows >= j of j's
    document; always complete when rows is None).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, hq, D = q.shape
    hk = k.shape[1]
    if k.shape != (N, hk, D) or v.shape != (N, hk, D) or hq % hk:
        raise ValueError("shape mismatch")
    G = hq // hk
    if do is not None:
        do = np.asarray(do, dtype=np.float64)
        if do.shape != q.shape:
            raise ValueError("do shape mismatch")
    doc, start = doc_tables(cu_seqlens, N)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)

    # row blocks sized so one [B, W] score matrix stays under max_block_elems
    # (document starts never decrease along the sequence, so the block's
    # first row has the smallest start)
    blocks = []
    i = 0
    while i < R:
        j = i + 1
        while j < R:
            width = (int(rows[j]) + 1 if causal else N) - int(start[rows[i]])
            if (j + 1 - i) * width > max_block_elems or j - i >= 1024:
                break
            j += 1
        blocks.append((i, j))
        i = j

    out_o = np.zeros((R, hq, D))
    out_lse = np.zeros((hq, R))
    res = {"rows": rows, "o": out_o, "lse": out_lse}
    if do is not None:
        res["delta"] = np.zeros((hq, R))
        res["dq"] = np.zeros((R, hq, D))
        res["dk"] = np.zeros((N, hk, D))
        res["dv"] = np.zeros((N, hk, D))

    items = [(h, b0, b1) for h in range(hq) for (b0, b1) in blocks]

    def run(item):
        h, b0, b1 = item
        return item, _block(h, rows[b0:b1], q, k, v, do, scale, G, doc, start, causal)

    if workers is None:
        workers = len(os.sched_getaffinity(0))
    if workers > 1 and len(items) > 1:
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(limits=1, user_api="blas")
        except Exception:  # pragma: no cover - threadpoolctl is optional
            limiter = None
        try:
            with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
                results = list(ex.map(run, items))
        finally:
            if limiter is not None:
                limiter.restore_original_limits()
    else:
        results = [run(it) for it in items]

    for (h, b0, b1), r in results:
        out_o[b0:b1, h, :] = r["o"]
        out_lse[h, b0:b1] = r["lse"]
        if do is not None:
            kvh = h // G
            res["delta"][h, b0:b1] = r["delta"]
            res["dq"][b0:b1, h, :] = r["dq"]
            res["dk"][r["lo"]:r["hi"], kvh, :] += r["dk"]
            res["dv"][r["lo"]:r["hi"], kvh, :] += r["dv"]
    return res


# ---------------------------------------------------------------------------
# merging attention results over disjoint key sets
# ---------------------------------------------------------------------------
def merge_ref(o_parts, lse_parts):
    """Attention over a union of disjoint key sets from the results over each
    set (the per-chunk results a ring of key/value chunks produces:
    "Snowflake's Ulysses trick ...", third paragraph, on Ring Attention).
    With c over the parts, per row i and head h:

        lse = log sum_c exp(lse_c),   o = sum_c exp(lse_c - lse) o_c.

    o_parts: arrays [N, hq, D]; lse_parts: arrays [hq, N] (natural log; -inf
    for a row with no visible key in that part). fp64. A row whose parts are
    all -inf gets o = 0 and lse = -inf."""
    lse_all = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])   # [C, hq, N]
    o_all = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])       # [C, N, hq, D]
    m = lse_all.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_all), np.exp(lse_all - m_safe[None]), 0.0)    # [C, hq, N]
    s = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, s, 1.0)), -np.inf)
    wn = np.where(finite[None], w / np.where(finite, s, 1.0)[None], 0.0)      # [C, hq, N]
    o = np.einsum("chn,cnhd->nhd", wn, o_all)
    return o, lse
