"""GPU parity of ulysses_pack / ulysses_unpack: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import sequence_parallelism_ulysses_amd as uly
import synthetic as syn
from oracle import (pack_heads_ref, pack_qkv_ref, pack_ref, replicated_kv_head, unpack_heads_ref,
                    unpack_qkv_ref, unpack_ref)
from harness import DEV, bits_to_dev, dev_to_bits

pytestmark = pytest.mark.gpu

CASES = [
    # (P, T, H, D, dtype)
    (4, 256, 8, 64, "f32"),      # c1 shards
    (8, 4096, 32, 128, "bf16"),  # c2 q/do shards
    (8, 4096, 8, 128, "bf16"),   # c2 k/v shards
    (3, 7, 6, 64, "bf16"),       # ragged: odd T, 2 heads per group
    (1, 5, 3, 128, "f32"),       # one rank: pack is a copy of the whole shard
    (5, 33, 15, 128, "bf16"),    # 3 heads per group
    (64, 2, 64, 64, "bf16"),     # the largest rank count
]


def _host_shards(P, T, H, D, dtype, seed):
    r = np.random.default_rng(seed)
    dt = np.uint16 if dtype == "bf16" else np.uint32
    return [r.integers(0, np.iinfo(dt).max, size=(T, H, D), dtype=dt, endpoint=True) for _ in range(P)]


@pytest.mark.parametrize("P,T,H,D,dtype", CASES)
def test_pack_unpack_bit_exact(P, T, H, D, dtype):
    # raw random bits (NaN payloads and denormals included) must survive
    host = _host_shards(P, T, H, D, dtype, seed=P * 1000 + T)
    dev = [bits_to_dev(s) for s in host]
    hh = H // P
    groups = sorted({0, P - 1, P // 2})
    for g in groups:
        out = torch.empty((P * T, hh, D), dtype=dev[0].dtype, device=DEV)
        uly.ulysses_pack(dev, g, out)
        torch.cuda.synchronize()
        want = pack_ref(host, g)
        assert np.array_equal(dev_to_bits(out), want), f"pack group {g}"
        # unpack into canary-filled shards: group heads restored, others untouched
        canary_bits = np.full((T, H, D), 0x7FA5 if dtype == "bf16" else 0x7FC0A5A5,
                              dtype=host[0].dtype)
        canary = [bits_to_dev(canary_bits.copy()) for _ in range(P)]
        uly.ulysses_unpack(out, g, canary)
        torch.cuda.synchronize()
        want_sh = unpack_ref(want, [canary_bits] * P, g)
        for j in range(P):
            assert np.array_equal(dev_to_bits(canary[j]), want_sh[j]), f"unpack group {g} shard {j}"


def test_pack_all_groups_roundtrip_c2():
    """Pack every group, unpack every group into zeros: the shards come back."""
    cfg = syn.CONFIGS["c2"]
    host = syn.all_shards_bits(cfg, "k")
    dev = [bits_to_dev(s) for s in host]
    back = [torch.zeros_like(s) for s in dev]
    for g in range(cfg.P):
        out = torch.empty((cfg.N, cfg.hk, cfg.D), dtype=torch.bfloat16, device=DEV)
        uly.ulysses_pack(dev, g, out)
        uly.ulysses_unpack(out, g, back)
    torch.cuda.synchronize()
    for a, b in zip(back, host):
        assert np.array_equal(dev_to_bits(a), b)


def test_pack_on_side_stream():
    """The call enqueues on the stream it is given."""
    host = _host_shards(4, 64, 8, 128, "bf16", seed=3)
    dev = [bits_to_dev(s) for s in host]
    out = torch.empty((256, 2, 128), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        uly.ulysses_pack(dev, 1, out)
    s.synchronize()
    assert np.array_equal(dev_to_bits(out), pack_ref(host, 1))


def test_pack_c4_q_shape_64bit_offsets():
    """Million-token case: the all-shards Q holds 2^32 elements, so offsets need
    64 bits. Check the last group on sampled tokens of every shard (including
    each shard's last token) against the oracle on those rows."""
    P, T, H, D = 8, 131072, 32, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20260313)
    dev = [torch.randint(-32768, 32767, (T, H, D), dtype=torch.int16, device=DEV, generator=gen).view(torch.bfloat16)
           for _ in range(P)]
    g = P - 1
    out = torch.empty((P * T, H // P, D), dtype=torch.bfloat16, device=DEV)
    uly.ulysses_pack(dev, g, out)
    torch.cuda.synchronize()
    ts = np.array([0, 1, 4095, 65536, T - 2, T - 1])
    mini = [dev_to_bits(s[torch.from_numpy(ts).to(DEV)]) for s in dev]   # [len(ts), H, D] per shard
    want = pack_ref(mini, g)                                             # rows j*len(ts) + i
    rows = np.concatenate([j * T + ts for j in range(P)])
    got = dev_to_bits(out[torch.from_numpy(rows).to(DEV)])
    assert np.array_equal(got, want)
    # and the inverse on the same buffers: write the group back into zeroed heads
    for s in dev:
        s.view(torch.int16)[:, g * 4:(g + 1) * 4, :] = 0
    uly.ulysses_unpack(out, g, dev)
    torch.cuda.synchronize()
    for j in range(P):
        assert np.array_equal(dev_to_bits(dev[j][torch.from_numpy(ts).to(DEV)]), mini[j])
    del dev, out
    torch.cuda.empty_cache()


def test_pack_rejects_mismatched_tensors():
    dev = [torch.zeros((8, 8, 64), dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    with pytest.raises(ValueError):
        uly.ulysses_pack(dev, 0, torch.zeros((32, 3, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(uly.UlyssesError):
        uly.ulysses_pack(dev, 4, torch.zeros((32, 2, 64), dtype=torch.bfloat16, device=DEV))


QKV_CASES = [
    # (P, T, Hq, Hkv, D, dtype)
    (8, 4096, 32, 8, 128, "bf16"),   # Llama-3.1-8B-shaped fused projection, 32k tokens over 8 ranks
    (4, 256, 8, 8, 64, "f32"),       # the tiny fp32 shapes
    (3, 37, 6, 3, 64, "bf16"),       # ragged: odd T, one kv head per group
    (1, 5, 4, 2, 128, "bf16"),       # one rank
    (2, 3000, 16, 4, 128, "bf16"),   # a partial last block in every section
    (64, 2, 64, 64, 64, "bf16"),     # the largest rank count
]


@pytest.mark.parametrize("P,T,Hq,Hkv,D,dtype", QKV_CASES)
def test_pack_unpack_qkv_bit_exact(P, T, Hq, Hkv, D, dtype):
    """Fused QKV pack and its inverse against the oracle, bit for bit, with
    random bit patterns; the inverse writes into canary-filled shards."""
    H = Hq + 2 * Hkv
    host = _host_shards(P, T, H, D, dtype, seed=7 * P + T)
    dev = [bits_to_dev(s) for s in host]
    tdt = dev[0].dtype
    hq, hk = Hq // P, Hkv // P
    for g in sorted({0, P - 1, P // 2}):
        outs = [torch.empty((P * T, c, D), dtype=tdt, device=DEV) for c in (hq, hk, hk)]
        uly.ulysses_pack_qkv(dev, Hq, Hkv, g, *outs)
        torch.cuda.synchronize()
        want = pack_qkv_ref(host, Hq, Hkv, g)
        for name, o, w in zip("qkv", outs, want):
            assert np.array_equal(dev_to_bits(o), w), f"pack_qkv {name} group {g}"
        canary_bits = np.full((T, H, D), 0x7FA5 if dtype == "bf16" else 0x7FC0A5A5, dtype=host[0].dtype)
        canary = [bits_to_dev(canary_bits.copy()) for _ in range(P)]
        uly.ulysses_unpack_qkv(*outs, Hq, Hkv, g, canary)
        torch.cuda.synchronize()
        want_sh = unpack_qkv_ref(*want, [canary_bits] * P, Hq, Hkv, g)
        for j in range(P):
            assert np.array_equal(dev_to_bits(canary[j]), want_sh[j]), f"unpack_qkv group {g} shard {j}"


def test_pack_qkv_equals_separate_packs():
    """The fused call and three ulysses_pack calls on the sections (strided
    views copied out) give the same bits (Llama-3.1-8B shapes, 128k tokens)."""
    P, T, Hq, Hkv, D = 8, 16384, 32, 8, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    dev = [torch.randint(-32768, 32767, (T, Hq + 2 * Hkv, D), dtype=torch.int16, device=DEV, generator=gen)
           .view(torch.bfloat16) for _ in range(P)]
    g = 3
    fused = [torch.empty((P * T, c, D), dtype=torch.bfloat16, device=DEV) for c in (4, 1, 1)]
    uly.ulysses_pack_qkv(dev, Hq, Hkv, g, *fused)
    bounds = [(0, Hq), (Hq, Hq + Hkv), (Hq + Hkv, Hq + 2 * Hkv)]
    for (a, b), f in zip(bounds, fused):
        sec = [s[:, a:b].contiguous() for s in dev]
        sep = torch.empty_like(f)
        uly.ulysses_pack(sec, g, sep)
        torch.cuda.synchronize()
        assert torch.equal(sep.view(torch.int16), f.view(torch.int16))
    # the oracle on sampled tokens of every shard (first, last, block edges)
    ts = np.array([0, 1, 8191, 8192, T - 2, T - 1])
    mini = [dev_to_bits(s[torch.from_numpy(ts).to(DEV)]) for s in dev]
    want = pack_qkv_ref(mini, Hq, Hkv, g)
    rows = torch.from_numpy(np.concatenate([j * T + ts for j in range(P)])).to(DEV)
    for f, w in zip(fused, want):
        assert np.array_equal(dev_to_bits(f[rows]), w)


MULTI_CASES = [
    # (P, T, head counts, D, dtype)
    (8, 4096, (32, 8, 8), 128, "bf16"),   # Q, K, V shards of the Llama-3.1-8B-shaped 32k workload
    (4, 256, (8, 8, 8), 64, "f32"),       # the tiny fp32 shapes
    (3, 37, (6, 3, 9), 64, "bf16"),       # ragged T, three different head counts
    (2, 3000, (16, 4), 128, "bf16"),      # two tensors, partial last blocks
    (1, 5, (4,), 128, "bf16"),            # one tensor, one rank
    (64, 2, (64, 64, 128), 64, "bf16"),   # the largest rank count
]


@pytest.mark.parametrize("P,T,heads,D,dtype", MULTI_CASES)
def test_pack_unpack_multi_bit_exact(P, T, heads, D, dtype):
    """Several tensors in one launch against the oracle tensor by tensor, bit
    for bit with random bit patterns; the inverse into canary-filled shards."""
    host = [_host_shards(P, T, H, D, dtype, seed=31 * i + T) for i, H in enumerate(heads)]
    dev = [[bits_to_dev(s) for s in h] for h in host]
    tdt = dev[0][0].dtype
    for g in sorted({0, P - 1, P // 2}):
        outs = [torch.empty((P * T, H // P, D), dtype=tdt, device=DEV) for H in heads]
        uly.ulysses_pack_multi(dev, g, outs)
        torch.cuda.synchronize()
        want = [pack_ref(h, g) for h in host]
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(dev_to_bits(o), w), f"pack_multi tensor {i} group {g}"
        canary_bits = [np.full((T, H, D), 0x7FA5 if dtype == "bf16" else 0x7FC0A5A5, dtype=host[0][0].dtype)
                       for H in heads]
        canary = [[bits_to_dev(c.copy()) for _ in range(P)] for c in canary_bits]
        uly.ulysses_unpack_multi(outs, g, canary)
        torch.cuda.synchronize()
        for i in range(len(heads)):
            want_sh = unpack_ref(want[i], [canary_bits[i]] * P, g)
            for j in range(P):
                assert np.array_equal(dev_to_bits(canary[i][j]), want_sh[j]), f"unpack_multi tensor {i} shard {j}"


HEADS_CASES = [
    # (P, T, H, D, dtype, [(head0, nheads), ...])
    (16, 2048, 8, 128, "bf16", [(replicated_kv_head(g, 16, 32, 8), 1) for g in (0, 1, 2, 7, 15)]),  # kv heads replicated
    (3, 37, 12, 64, "bf16", [(3, 5), (0, 12), (11, 1)]),     # any run of heads, ragged T
    (4, 256, 8, 64, "f32", [(2, 2), (5, 3)]),                 # fp32
    (64, 2, 4, 128, "bf16", [(1, 2)]),                        # more ranks than heads
]


@pytest.mark.parametrize("P,T,H,D,dtype,runs", HEADS_CASES)
def test_pack_unpack_heads_bit_exact(P, T, H, D, dtype, runs):
    """Head runs (including the replicated kv head of a rank when there are
    fewer kv heads than ranks) against the oracle bit for bit; the inverse
    into canary-filled shards."""
    host = _host_shards(P, T, H, D, dtype, seed=13 * P + T)
    dev = [bits_to_dev(s) for s in host]
    for h0, nh in runs:
        out = torch.empty((P * T, nh, D), dtype=dev[0].dtype, device=DEV)
        uly.ulysses_pack_heads(dev, h0, nh, out)
        torch.cuda.synchronize()
        want = pack_heads_ref(host, h0, nh)
        assert np.array_equal(dev_to_bits(out), want), f"pack_heads [{h0}, +{nh})"
        canary_bits = np.full((T, H, D), 0x7FA5 if dtype == "bf16" else 0x7FC0A5A5, dtype=host[0].dtype)
        canary = [bits_to_dev(canary_bits.copy()) for _ in range(P)]
        uly.ulysses_unpack_heads(out, h0, nh, canary)
        torch.cuda.synchronize()
        want_sh = unpack_heads_ref(want, [canary_bits] * P, h0, nh)
        for j in range(P):
            assert np.array_equal(dev_to_bits(canary[j]), want_sh[j]), f"unpack_heads shard {j}"


@pytest.mark.parametrize("T", [16384, 131072])
def test_pack_unpack_multi_full_size_sampled(T):
    """The step's regrouping of Q, K, V (32, 8, 8 heads over 8 ranks) in one
    launch at 128k and 1M tokens (the all-shards Q of the latter holds 2^32
    elements): the last group, checked on sampled tokens of every shard
    against the oracle; then the inverse into zeroed heads."""
    P, D, g = 8, 128, 7
    heads = (32, 8, 8)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(T + 17)
    dev = [[torch.randint(-32768, 32767, (T, H, D), dtype=torch.int16, device=DEV, generator=gen).view(torch.bfloat16)
            for _ in range(P)] for H in heads]
    outs = [torch.empty((P * T, H // P, D), dtype=torch.bfloat16, device=DEV) for H in heads]
    uly.ulysses_pack_multi(dev, g, outs)
    torch.cuda.synchronize()
    ts = np.array([0, 1, 4095, T // 2, T - 2, T - 1])
    idx = torch.from_numpy(ts).to(DEV)
    rows = torch.from_numpy(np.concatenate([j * T + ts for j in range(P)])).to(DEV)
    minis = []
    for i, H in enumerate(heads):
        mini = [dev_to_bits(s[idx]) for s in dev[i]]
        minis.append(mini)
        assert np.array_equal(dev_to_bits(outs[i][rows]), pack_ref(mini, g)), f"tensor {i}"
    hh = [H // P for H in heads]
    for i in range(len(heads)):
        for s in dev[i]:
            s.view(torch.int16)[:, g * hh[i]:(g + 1) * hh[i], :] = 0
    uly.ulysses_unpack_multi(outs, g, dev)
    torch.cuda.synchronize()
    for i in range(len(heads)):
        for j in range(P):
            assert np.array_equal(dev_to_bits(dev[i][j][idx]), minis[i][j]), f"unpack tensor {i} shard {j}"
    del dev, outs
    torch.cuda.empty_cache()
