"""Calls of random shape for the gather + upconvert, the merge of partial
results and the page re-split, against their oracles: byte for byte for the
gather and the re-split, to the merge's arithmetic bound for the merge."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from oracle import gather as oracle_gather
from oracle import merge as oracle_merge
from oracle import pages as oracle_pages
from tests.gpu_util import DEV, bf16_dev, build_cache, to_f64

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("seed", range(16))
def test_gather_random_calls(seed):
    """Row counts from 0 to 5,000, rope 0 or 64, a destination wider than 576
    columns or not, slot lists with slot 0, repeats and invalid entries."""
    rng = np.random.default_rng(500 + seed)
    rope_dim = int(rng.choice([0, 64]))
    num_slots = int(rng.choice([64, 1000, 4096]))
    n = int(rng.choice([0, 1, 2, 63, 64, 65, 777, 5000]))
    extra = int(rng.choice([0, 0, 8, 64]))
    print(f"gather sweep seed={seed} rope={rope_dim} slots={num_slots} n={n} extra={extra}", flush=True)
    lat, rope, slots_all = wl.cache_rows(rng, num_slots, rope_dim)
    x = wl.f32_from_bf16_bits(lat) * np.exp2(rng.integers(-30, 30, size=(lat.shape[0], 1)))
    lat = wl.bf16_bits_from_f32(x.astype(np.float32))
    cfg = dict(num_slots=num_slots, rope_dim=rope_dim, latent=lat, rope=rope, slots=slots_all,
               slot0=wl.slot0_bytes(rng, str(rng.choice(["ff", "zero", "random"]))))
    cache = build_cache(cfg)
    slots = rng.integers(0, num_slots, size=n).astype(np.int64)
    bad = rng.random(n) < 0.1
    slots[bad] = rng.choice([-1, -5, num_slots, num_slots + 3, 1 << 40], size=int(bad.sum()))
    want = oracle_gather.gather_upconvert(cache.cpu().numpy(), slots, rope_dim)
    if extra:
        full = torch.full((n, 576 + extra), float("nan"), dtype=torch.bfloat16, device=DEV)
        out = full[:, :576]
        smla.gather_upconvert(cache, torch.from_numpy(slots).to(DEV), rope_dim, out=out)
        torch.cuda.synchronize()
        assert bool(torch.isnan(full[:, 576:].float()).all()), "columns past 576 were written"
        got = _bits(out.contiguous())
    else:
        out = smla.gather_upconvert(cache, torch.from_numpy(slots).to(DEV), rope_dim)
        torch.cuda.synchronize()
        got = _bits(out)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(16))
def test_merge_random_calls(seed):
    """P from 1 to 40 parts, T and H ragged, empty parts (lse = -inf, NaN
    outputs that must not be read) and (row, head) pairs with every part empty."""
    rng = np.random.default_rng(600 + seed)
    P = int(rng.choice([1, 2, 3, 7, 8, 9, 16, 17, 40]))
    T = int(rng.choice([1, 2, 5, 33, 130]))
    H = int(rng.choice([1, 3, 16, 17, 64]))
    T = max(1, min(T, 16384 // (P * H)))         # keeps the float64 oracle small
    print(f"merge sweep seed={seed} P={P} T={T} H={H}", flush=True)
    o = wl.normal_bf16(rng, (P, T, H, 512))
    l = rng.uniform(-30.0, 30.0, size=(P, T, H)).astype(np.float32)
    empty = rng.random((P, T, H)) < float(rng.choice([0.0, 0.3, 0.9]))
    l[empty] = -np.inf
    o[empty] = 0x7FC0
    out, lse = smla.merge(bf16_dev(o), torch.from_numpy(l).to(DEV))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_merge.merge(oracle_merge.bf16_to_f64(o), l.astype(np.float64))
    g = to_f64(out)
    assert np.all(np.isfinite(g))
    live = ~empty
    omax = np.abs(oracle_merge.bf16_to_f64(o))[live].max() if live.any() else 0.0
    # fp32 weights and sums (~1e-6 relative), then one bf16 rounding (2^-9)
    assert np.all(np.abs(g - ref_out) <= 2.0**-8 * np.abs(ref_out) + 1e-5 * omax)
    gl = lse.cpu().numpy().astype(np.float64)
    inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(gl), inf)
    if (~inf).any():
        assert np.abs(gl[~inf] - ref_lse[~inf]).max() <= 1e-5 * max(1.0, np.abs(ref_lse[~inf]).max())
    assert np.all(g[inf] == 0.0)


@pytest.mark.parametrize("seed", range(12))
def test_split_pages_random_calls(seed):
    """Random pools, page lists with repeats and invalid entries, row formats and
    destination paddings; the destination keeps its zero fill where no page
    lands."""
    rng = np.random.default_rng(800 + seed)
    row_bytes = int(rng.choice([656, 1024, 1152, 585]))
    pad = int(rng.choice([0, 16, 48]))
    n_src = int(rng.choice([1, 5, 37]))
    n = int(rng.choice([0, 1, 7, 40]))
    print(f"split sweep seed={seed} rb={row_bytes} pad={pad} src={n_src} n={n}", flush=True)
    pool = rng.integers(0, 256, size=(n_src, 256 * row_bytes), dtype=np.uint8)
    pages = rng.integers(0, n_src, size=n).astype(np.int32)
    bad = rng.random(n) < 0.15
    pages[bad] = rng.choice([-1, n_src, n_src + 9, 2**31 - 1], size=int(bad.sum())).astype(np.int32)
    dst_h = np.zeros((4 * n_src, 64 * row_bytes + pad), dtype=np.uint8)
    dst = torch.from_numpy(dst_h).to(DEV)
    smla.split_pages_64(torch.from_numpy(pool).to(DEV), torch.from_numpy(pages).to(DEV), dst, row_bytes)
    torch.cuda.synchronize()
    oracle_pages.split_pages_64(pool, pages, dst_h, row_bytes)
    assert np.array_equal(dst.cpu().numpy(), dst_h)
