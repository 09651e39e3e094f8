"""Pins of the oracle's sparse attention: dense causal attention through torch's
SDPA on library-decoded values, closed forms, invariances, and the pages'
clamp-to-slot-0 failure pattern as a negative control."""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as A
from oracle import writer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot0_harness.txt")


def _cache(num_slots, rope_dim, seed, slot0="zero"):
    rng = np.random.default_rng(seed)
    lat, rope, slots = wl.cache_rows(rng, num_slots, rope_dim)
    cache = np.zeros((num_slots, 656), dtype=np.uint8)
    writer.kv_write(cache, lat, rope, slots)
    cache[0] = wl.slot0_bytes(rng, slot0)
    return cache


def _lib_k(cache, slots, rope_dim):
    """K rows decoded with torch's float8_e4m3fn / bfloat16 casts (not the oracle's table)."""
    rows = torch.from_numpy(cache[np.asarray(slots)].copy())
    codes = rows[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    sc = rows[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
    k = (codes.view(-1, 4, 128) * sc[:, :, None]).reshape(-1, 512)
    if rope_dim:
        pe = rows[:, 528:528 + 2 * rope_dim].contiguous().view(torch.bfloat16).to(torch.float64)
        k = torch.cat([k, pe], dim=1)
    return k


def _lib_q(q_bits):
    return torch.from_numpy(q_bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64)


@pytest.mark.parametrize("rope_dim", [64, 0])
def test_dense_causal_matches_sdpa(rope_dim):
    """When the top-k lists cover the whole causal context, sparse attention is
    dense causal attention; compared with torch SDPA in float64."""
    rng = np.random.default_rng(11)
    num_slots, T, H, W = 4096, 70, 4, 128
    cache = _cache(num_slots, rope_dim, 12, slot0="ff")
    idx, seq = wl.prefill_topk(rng, T, W, num_slots)
    q = wl.normal_bf16(rng, (T, H, 512 + rope_dim))
    sm = 1.0 / np.sqrt(512 + rope_dim)
    out, lse = A.sparse_mla_attn(q, cache, idx, W, rope_dim, sm)
    k = _lib_k(cache, seq, rope_dim)                          # [T][D] in sequence order
    qt = _lib_q(q).permute(1, 0, 2)                           # [H][T][D]
    kk = k[None].expand(H, T, -1)
    vv = k[None, :, :512].expand(H, T, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kk, vv, is_causal=True, scale=sm)
    ref = ref.permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    s = sm * torch.einsum("htd,sd->hts", qt, k)
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -np.inf)
    ref_lse = torch.logsumexp(s, dim=2).permute(1, 0).numpy()
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def test_closed_forms():
    cache = _cache(512, 64, 13, slot0="ff")
    rng = np.random.default_rng(14)
    q = wl.normal_bf16(rng, (5, 3, 576))
    sm = 1.0 / 24.0
    a, b = 17, 300
    idx = np.full((5, 8), -1, dtype=np.int32)
    idx[0, 5] = a                         # one entry
    idx[1, [1, 6]] = [a, b]               # two entries
    idx[2, [0, 3]] = [a, a]               # a duplicated entry
    idx[4, 2:7] = [3, 9, 27, 81, 243]     # q = 0 below: plain mean
    q[4] = 0
    out, lse = A.sparse_mla_attn(q, cache, idx, 8, 64, sm)
    k = _lib_k(cache, [a, b, 3, 9, 27, 81, 243], 64).numpy()
    qf = _lib_q(q).numpy()
    sa, sb = sm * qf[:, :, :] @ k[0], sm * qf @ k[1]
    assert np.array_equal(out[0], np.broadcast_to(k[0, :512], (3, 512)))
    assert np.allclose(lse[0], sa[0], rtol=0, atol=1e-13)
    p = 1.0 / (1.0 + np.exp(sb[1] - sa[1]))
    assert np.allclose(out[1], p[:, None] * k[0, :512] + (1 - p)[:, None] * k[1, :512], atol=1e-13)
    assert np.allclose(out[2], out[0], atol=1e-15)
    assert np.allclose(lse[2], sa[2] + np.log(2.0), atol=1e-13)
    assert np.array_equal(out[3], np.zeros((3, 512))) and np.all(lse[3] == -np.inf)
    assert np.allclose(out[4], np.broadcast_to(k[2:, :512].mean(axis=0), (3, 512)), atol=1e-13)
    assert np.allclose(lse[4], np.log(5.0), atol=1e-14)


def _tiny():
    c = wl.config_tiny()
    cache = np.zeros((c["num_slots"], 656), dtype=np.uint8)
    writer.kv_write(cache, c["latent"], c["rope"], c["slots"])
    cache[0] = c["slot0"]
    return c, cache


def test_permutation_invariance():
    c, cache = _tiny()
    out, lse = A.sparse_mla_attn(c["q"], cache, c["idx"], c["W"], 64, c["sm_scale"])
    rng = np.random.default_rng(15)
    idx2 = np.stack([rng.permutation(r) for r in c["idx"]])   # -1s move into the middle
    out2, lse2 = A.sparse_mla_attn(c["q"], cache, idx2, c["W"], 64, c["sm_scale"])
    assert np.allclose(out, out2, rtol=0, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)


def test_slot0_and_unreferenced_bytes_do_not_matter():
    c, cache = _tiny()
    ref = A.sparse_mla_attn(c["q"], cache, c["idx"], c["W"], 64, c["sm_scale"])
    used = set(c["idx"][c["idx"] >= 0].tolist())
    unused = np.array([s for s in range(1, c["num_slots"]) if s not in used])
    rng = np.random.default_rng(16)
    for poison in ("ff", "7f", "random", "zero"):
        cache2 = cache.copy()
        cache2[0] = wl.slot0_bytes(rng, poison)
        cache2[unused] = rng.integers(0, 256, size=(unused.size, 656), dtype=np.uint8)
        got = A.sparse_mla_attn(c["q"], cache2, c["idx"], c["W"], 64, c["sm_scale"])
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        assert np.all(np.isfinite(got[0]))


def test_width_is_capacity_and_out_of_range_is_padding():
    c, cache = _tiny()
    W = c["W"]
    base = A.sparse_mla_attn(c["q"], cache, c["idx"], W, 64, c["sm_scale"])
    wide = np.full((2, W + 128), -1, dtype=np.int32)
    wide[:, :W] = c["idx"]
    got = A.sparse_mla_attn(c["q"], cache, wide, W + 128, 64, c["sm_scale"])
    assert np.array_equal(got[0], base[0])
    beyond = wide.copy()
    beyond[:, W:] = 5                       # entries past the width are not part of the row
    got = A.sparse_mla_attn(c["q"], cache, beyond, W, 64, c["sm_scale"])
    assert np.array_equal(got[0], base[0])
    oor = c["idx"].copy()
    oor[oor == -1] = c["num_slots"]         # >= num_slots counts as padding
    got = A.sparse_mla_attn(c["q"], cache, oor, W, 64, c["sm_scale"])
    assert np.array_equal(got[0], base[0])


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            kind, T, poison, neg, nan = line.split()
            rows.append((kind, int(T), poison, int(neg), int(nan)))
    return rows


@pytest.mark.parametrize("case", _golden(), ids=lambda r: f"{r[0]}-T{r[1]}-{r[2]}")
def test_negative_control_reproduces_page_pattern(case):
    """The clamp-to-slot-0 reader yields NaN in exactly the rows that carry a -1
    when slot 0 holds 0xFF, and none with zeros; the oracle never does."""
    kind, T, poison, n_neg, n_nan = case
    H, num_slots = 16, 64 * 64                 # one 64-page cache
    W = n_neg + 1                              # rows t < W-1 carry -1 padding
    rng = np.random.default_rng(17 + T)
    cache = _cache(num_slots, 64, 18)
    cache[0] = wl.slot0_bytes(rng, poison)
    idx, _ = wl.prefill_topk(rng, T, W, num_slots)
    assert int((idx < 0).any(axis=1).sum()) == n_neg
    q = wl.normal_bf16(rng, (T, H, 576))
    bad = A.clamped_gather_attn(q, cache, idx, W, 64, 1 / 24)
    nan_rows = np.nonzero(~np.isfinite(bad).all(axis=(1, 2)))[0]
    assert nan_rows.size == n_nan
    if n_nan:
        assert np.array_equal(nan_rows, np.nonzero((idx < 0).any(axis=1))[0])
        assert int((~np.isfinite(bad)).sum()) == n_nan * H * 512
    good, lse = A.sparse_mla_attn(q, cache, idx, W, 64, 1 / 24)
    assert np.all(np.isfinite(good)) and np.all(np.isfinite(lse))
