"""The seeded input generators: determinism, shapes, bf16 rounding, documents."""
import numpy as np
import torch

import synthetic as syn


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even, checked against torch's float32 -> bfloat16 cast."""
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 65504.0, 1e-20], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(syn.f32_to_bf16_bits(x), want)
    assert np.array_equal(syn.bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_shards_deterministic_and_independent():
    c = syn.CONFIGS["c1"]
    a = syn.shard_bits(c, "q", 2)
    b = syn.shard_bits(c, "q", 2)
    assert a.dtype == np.uint32 and a.shape == (256, 8, 64)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, syn.shard_bits(c, "q", 1))
    assert not np.array_equal(a, syn.shard_bits(c, "k", 2))
    vals = syn.shard_values(c, "q", 2)
    assert abs(vals.mean()) < 0.02 and abs(vals.std() - 1) < 0.02


def test_bf16_config_shapes():
    c = syn.CONFIGS["c2"]
    assert (c.T, c.hq, c.hk) == (4096, 4, 1)
    s = syn.shard_bits(c, "k", 0)
    assert s.dtype == np.uint16 and s.shape == (4096, 8, 128)


def test_cu_seqlens_lognormal():
    c = syn.CONFIGS["c5"]
    cu = syn.cu_seqlens(c)
    assert cu[0] == 0 and cu[-1] == c.N and cu.dtype == np.int32
    lens = np.diff(cu)
    assert np.all(lens[:-1] >= 128) and np.all(lens <= 32768) and lens[-1] >= 1
    assert np.array_equal(cu, syn.cu_seqlens(c))
    assert syn.cu_seqlens(syn.CONFIGS["c2"]) is None
