"""Pins of the oracle's BF16-cache writer and attention: torch's own scaled
dot-product attention on the same bf16 rows, agreement with the quantised-cache
oracle where the two caches hold the same values, and the writer's slot rule."""
import numpy as np
import torch

import workloads as wl
from oracle import attention as A
from oracle import writer


def _bf16_cache(rng, num_slots, rope_dim):
    lat, rope, slots = wl.cache_rows(rng, num_slots, rope_dim)
    cache = np.zeros((num_slots, 512 + rope_dim), dtype=np.uint16)
    writer.kv_write_bf16(cache, lat, rope, slots)
    cache[0] = 0x7FC0                                   # NaN row in the reserved slot
    return cache


def test_matches_torch_sdpa_on_the_same_rows():
    rng = np.random.default_rng(11)
    for rope_dim in (0, 64):
        cache = _bf16_cache(rng, 600, rope_dim)
        T, H, W = 3, 4, 160
        q = wl.normal_bf16(rng, (T, H, 512 + rope_dim))
        idx = np.full((T, W), -1, dtype=np.int32)
        for t in range(T):
            pos = rng.choice(W, size=100 + 20 * t, replace=False)
            idx[t, pos] = rng.choice(np.arange(1, 600), size=pos.size, replace=False)
        sm = 1.0 / np.sqrt(512 + rope_dim)
        out, lse = A.sparse_mla_attn_bf16(q, cache, idx, W, rope_dim, sm)
        qt = torch.from_numpy(q.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
        for t in range(T):
            v = idx[t][idx[t] >= 0]
            k = torch.from_numpy(cache[v].astype(np.int16)).view(torch.bfloat16).to(torch.float64)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt[t][:, None, :], k[None].expand(H, -1, -1), k[None, :, :512].expand(H, -1, -1),
                scale=sm)[:, 0]                          # heads as the batch, one query each
            assert np.abs(out[t] - ref.numpy()).max() < 1e-12
            s = sm * (qt[t] @ k.T)
            assert np.abs(lse[t] - torch.logsumexp(s, dim=1).numpy()).max() < 1e-12


def test_agrees_with_the_quantised_oracle_on_equal_values():
    """Rows whose values are e4m3 codes with |max| = 448 per tile quantise with
    scale 1 exactly, so the fp8 cache dequantises to the very bf16 values."""
    rng = np.random.default_rng(12)
    num_slots = 300
    from oracle import e4m3
    codes = rng.integers(0, 256, size=(num_slots - 1, 512), dtype=np.int64).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10                # no NaN codes
    codes[:, ::128] = 0x7E                               # each tile holds +448: scale = 1
    vals = e4m3.decode(codes).astype(np.float32)
    lat = wl.bf16_bits_from_f32(vals)
    assert np.array_equal(wl.f32_from_bf16_bits(lat), vals)   # e4m3 values are bf16 values
    slots = np.arange(1, num_slots, dtype=np.int64)
    q8 = np.zeros((num_slots, 656), dtype=np.uint8)
    writer.kv_write(q8, lat, None, slots)
    qb = np.zeros((num_slots, 512), dtype=np.uint16)
    writer.kv_write_bf16(qb, lat, None, slots)
    q = wl.normal_bf16(rng, (2, 4, 512))
    idx = np.stack([rng.choice(np.arange(1, num_slots), size=64, replace=False) for _ in range(2)]).astype(np.int32)
    o8, l8 = A.sparse_mla_attn(q, q8, idx, 64, 0, 0.05)
    ob, lb = A.sparse_mla_attn_bf16(q, qb, idx, 64, 0, 0.05)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_writer_slot_rule():
    rng = np.random.default_rng(13)
    lat = wl.normal_bf16(rng, (6, 512))
    lat[3] = 0x7FC0                                      # a padding row's NaN inputs
    cache = np.full((10, 512), 0xA5A5, dtype=np.uint16)
    keep = writer.kv_write_bf16(cache, lat, None, np.array([4, 0, 9, 0, -1, 12]))
    assert keep.tolist() == [True, False, True, False, False, False]
    assert np.array_equal(cache[4], lat[0]) and np.array_equal(cache[9], lat[2])
    untouched = [i for i in range(10) if i not in (4, 9)]
    assert np.all(cache[untouched] == 0xA5A5)
