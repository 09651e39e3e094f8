"""HIP gather + upconvert vs the oracle, byte for byte: RoPE and NoPE rows,
sentinel bytes in the NoPE tail, invalid entries and the poisoned slot 0,
ragged row counts into a wider row-strided destination, the bench-sized
gather (sampled rows) and a cache beyond 4 GiB."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from oracle import gather as oracle_gather
from tests.gpu_util import DEV, build_cache

pytestmark = pytest.mark.gpu


def _small_cfg(rope_dim, seed, num_slots=4096):
    rng = np.random.default_rng(seed)
    lat, rope, slots = wl.cache_rows(rng, num_slots, rope_dim)
    # rows spanning many binades, so scales and products cover the range
    x = wl.f32_from_bf16_bits(lat) * np.exp2(rng.integers(-40, 40, size=(lat.shape[0], 1)))
    lat = wl.bf16_bits_from_f32(x.astype(np.float32))
    return rng, dict(num_slots=num_slots, rope_dim=rope_dim, latent=lat, rope=rope, slots=slots,
                     slot0=wl.slot0_bytes(rng, "ff"))


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rope_dim", [64, 0])
def test_gather_byte_exact(rope_dim):
    print(f"gather rope={rope_dim}", flush=True)
    rng, cfg = _small_cfg(rope_dim, 11 + rope_dim)
    cache = build_cache(cfg)
    if rope_dim == 0:
        cache[1:, 528:] = 0xA5            # sentinel tails must never reach the output
    cache[17, 3] = 0x7F                   # NaN codes inside an ordinary row
    cache[17, 200] = 0xFF
    slots = rng.integers(1, cfg["num_slots"], size=3001).astype(np.int64)
    slots[::97] = -1
    slots[5] = cfg["num_slots"]
    slots[7] = 1 << 40
    slots[9] = 0                          # slot 0 (0xFF bytes) is read like any slot
    slots[11] = 17
    out = smla.gather_upconvert(cache, torch.from_numpy(slots).to(DEV), rope_dim)
    torch.cuda.synchronize()
    want = oracle_gather.gather_upconvert(cache.cpu().numpy(), slots, rope_dim)
    assert np.array_equal(_bits(out), want)
    if rope_dim == 0:
        assert np.all(_bits(out)[:, 512:] == 0)


@pytest.mark.parametrize("n", [1, 3, 257])
def test_ragged_rows_into_a_strided_destination(n):
    rng, cfg = _small_cfg(64, 21, num_slots=1024)
    cache = build_cache(cfg)
    slots = rng.integers(-2, cfg["num_slots"] + 2, size=n).astype(np.int64)
    dst = torch.full((n, 640), -7.0, dtype=torch.bfloat16, device=DEV)
    smla.gather_upconvert(cache, torch.from_numpy(slots).to(DEV), 64, out=dst)
    torch.cuda.synchronize()
    got = _bits(dst)
    want = oracle_gather.gather_upconvert(cache.cpu().numpy(), slots, 64)
    assert np.array_equal(got[:, :576], want)
    assert bool(torch.all(dst[:, 576:] == -7.0))     # columns past 576 untouched


def test_bench_sized_gather_sampled():
    """65,536 distinct slots of a 131,072-slot NoPE cache (the timed shape)."""
    cfg = wl.config_nope_decode(1)
    cache = build_cache(cfg, check_slots=np.arange(1, 4096))
    rng = np.random.default_rng(5)
    slots = rng.choice(np.arange(1, cfg["num_slots"]), size=65536, replace=False).astype(np.int64)
    out = smla.gather_upconvert(cache, torch.from_numpy(slots).to(DEV), 0)
    torch.cuda.synchronize()
    pick = rng.choice(65536, size=2048, replace=False)
    rows = cache[torch.from_numpy(slots[pick]).to(DEV)].cpu().numpy()
    want = oracle_gather.gather_upconvert(rows, np.arange(len(pick)), 0)
    assert np.array_equal(_bits(out)[pick], want)


def test_cache_beyond_4_gib():
    num_slots = 7_000_000                 # 4.59 GB of rows
    rng = np.random.default_rng(9)
    cache = torch.zeros((num_slots, 656), dtype=torch.uint8, device=DEV)
    slots = np.concatenate([rng.integers(6_600_000, num_slots, size=500),
                            rng.integers(1, 1000, size=100)]).astype(np.int64)
    uniq = np.unique(slots)
    lat = wl.normal_bf16(rng, (uniq.size, 512))
    pe = wl.normal_bf16(rng, (uniq.size, 64))
    from tests.gpu_util import bf16_dev
    smla.kv_write(bf16_dev(lat), bf16_dev(pe), torch.from_numpy(uniq).to(DEV), cache)
    out = smla.gather_upconvert(cache, torch.from_numpy(slots).to(DEV), 64)
    torch.cuda.synchronize()
    rows = cache[torch.from_numpy(slots).to(DEV)].cpu().numpy()
    want = oracle_gather.gather_upconvert(rows, np.arange(slots.size), 64)
    assert np.array_equal(_bits(out), want)
