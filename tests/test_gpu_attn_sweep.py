"""Attention over calls of random shape against the float64 oracle.

Each call draws rope 0 or 64, T, H and the buffer width W across the launch
plan's boundaries (one or many splits, two or three merged inside the launch,
the merge kernels, four-wavefront workgroups, buffers wider than one scan, row
strides wider than W), over a small cache whose top-k rows mix empty, full and
partial rows with padding anywhere, repeated slots, slot 0 and out-of-range
entries; fp8 and BF16 caches.  Sampled rows meet the parity bar; every row is
finite, and rows without a valid entry give zeros and -inf.  Each fp8 call is
made twice, on workspaces of 0xA5 bytes and of zeros, and must give the same
bits both times.

SMLA_SWEEP_SEEDS (default 96) sets how many fp8 shapes are drawn; a long run
with 8,000 takes about eight minutes on one GPU."""
import os

import numpy as np
import pytest
import torch

import sparse_mla_attention_fp8_amd as smla
import workloads as wl
from tests.gpu_util import DEV, assert_parity, bf16_dev, build_cache, oracle_for

pytestmark = pytest.mark.gpu

SEEDS = int(os.environ.get("SMLA_SWEEP_SEEDS", "96"))


@pytest.mark.parametrize("seed", range(SEEDS))
def test_random_shape(seed):
    _check_random_call(wl.config_random_shape(seed), seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_many_heads(seed):
    """64 to 128 heads: several head groups per row, in every plan kind."""
    _check_random_call(wl.config_random_shape_many_heads(seed), seed)


def _check_random_call(cfg, seed):
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    print(f"sweep seed={seed} rope={cfg['rope_dim']} T={T} H={H} W={W} "
          f"slots={cfg['num_slots']} stride+{cfg['stride_extra']}", flush=True)
    cache = build_cache(cfg)
    idx = cfg["idx"]
    q = bf16_dev(cfg["q"])
    it = torch.from_numpy(idx).to(DEV)
    need = max(smla.workspace_size(T, H, W, cfg["rope_dim"]), 16)
    res = []
    for fill in (0xA5, 0):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        res.append(smla.attn(q, cache, it, cfg["sm_scale"], cfg["rope_dim"], topk_capacity=W, workspace=ws))
    torch.cuda.synchronize()
    (out, lse), (out2, lse2) = res
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "bits differ between calls"

    o = out.float()
    assert bool(torch.isfinite(o).all()), "non-finite output"
    active = idx[:, :W]
    valid = (active >= 0) & (active < cfg["num_slots"])
    empty = np.nonzero(~valid.any(axis=1))[0]
    if empty.size:
        e = torch.from_numpy(empty).to(DEV)
        assert bool((o[e] == 0).all()) and bool(torch.isneginf(lse[e]).all())

    rng = np.random.default_rng(seed)
    rows = {0, T - 1} | set(rng.choice(T, size=min(T, 4), replace=False).tolist())
    if empty.size:
        rows.add(int(empty[0]))
    rows = sorted(rows)
    ref_out, ref_lse = oracle_for(cfg, rows, idx=idx, W=W)
    assert_parity(out, lse, ref_out, ref_lse, rows)


@pytest.mark.parametrize("seed", range(32))
def test_random_shape_bf16_cache(seed):
    """The same sweep over a BF16 cache written by the BF16 writer (slot 0 a
    NaN row unless the lists name it, then zeros)."""
    from oracle import attention as oracle_attn

    cfg = wl.config_random_shape(1000 + seed)
    T, H, W, rope_dim, num_slots = cfg["T"], cfg["H"], cfg["W"], cfg["rope_dim"], cfg["num_slots"]
    print(f"bf16 sweep seed={seed} rope={rope_dim} T={T} H={H} W={W} slots={num_slots}", flush=True)
    width = 512 + rope_dim
    cache = torch.zeros((num_slots, width), dtype=torch.bfloat16, device=DEV)
    smla.kv_write_bf16(bf16_dev(cfg["latent"]), bf16_dev(cfg["rope"]) if rope_dim else None,
                       torch.from_numpy(cfg["slots"]).to(DEV), cache)
    if cfg["slot0"].any():
        cache[0] = float("nan")
    idx = cfg["idx"]
    out, lse = smla.attn_bf16(bf16_dev(cfg["q"]), cache, torch.from_numpy(idx).to(DEV), cfg["sm_scale"],
                              topk_capacity=W)
    torch.cuda.synchronize()

    o = out.float()
    assert bool(torch.isfinite(o).all()), "non-finite output"
    active = idx[:, :W]
    empty = np.nonzero(~((active >= 0) & (active < num_slots)).any(axis=1))[0]
    if empty.size:
        e = torch.from_numpy(empty).to(DEV)
        assert bool((o[e] == 0).all()) and bool(torch.isneginf(lse[e]).all())

    rng = np.random.default_rng(seed)
    rows = {0, T - 1} | set(rng.choice(T, size=min(T, 4), replace=False).tolist())
    if empty.size:
        rows.add(int(empty[0]))
    rows = sorted(rows)
    host = cache.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_out, ref_lse = oracle_attn.sparse_mla_attn_bf16(cfg["q"], host, idx, W, rope_dim, cfg["sm_scale"],
                                                        rows=rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)
