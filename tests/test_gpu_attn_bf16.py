"""HIP BF16-cache writer and attention vs the float64 oracle: the writer byte
for byte (slot rule, NaN padding rows), attention on NoPE and RoPE decode rows
with splits and a merge, padding anywhere, empty rows and out-of-range
entries, a NaN row in the reserved slot, head counts, prefill rows, the
full-size decode batches (sampled rows) and caches beyond 4 GiB."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from oracle import attention as oracle_attn
from oracle import writer as oracle_writer
from tests.gpu_util import DEV, assert_parity, bf16_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _build(cfg, check=True):
    """BF16 cache written by the HIP writer (checked against the oracle), slot 0 = NaN row."""
    width = 512 + cfg["rope_dim"]
    rope = cfg["rope"] if cfg["rope_dim"] else None
    cache = torch.zeros((cfg["num_slots"], width), dtype=torch.bfloat16, device=DEV)
    smla.kv_write_bf16(bf16_dev(cfg["latent"]), None if rope is None else bf16_dev(rope),
                       torch.from_numpy(cfg["slots"]).to(DEV), cache)
    torch.cuda.synchronize()
    if check:
        host = np.zeros((cfg["num_slots"], width), dtype=np.uint16)
        oracle_writer.kv_write_bf16(host, cfg["latent"], rope, cfg["slots"])
        assert np.array_equal(_bits(cache), host)
    cache[0] = torch.from_numpy(np.full(width, 0x7FC0, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)
    return cache


def _oracle(cfg, cache, idx, rows):
    need = idx[list(rows)].ravel()
    need = np.unique(need[(need >= 0) & (need < cfg["num_slots"])])
    host = np.zeros((cfg["num_slots"], cache.shape[1]), dtype=np.uint16)
    host[need] = _bits(cache[torch.from_numpy(need).to(DEV)])
    return oracle_attn.sparse_mla_attn_bf16(cfg["q"], host, idx, idx.shape[1], cache.shape[1] - 512,
                                            cfg["sm_scale"], rows=list(rows))


def _run(cfg, cache, idx, W=None):
    out, lse = smla.attn_bf16(bf16_dev(cfg["q"]), cache, torch.from_numpy(np.ascontiguousarray(idx)).to(DEV),
                              cfg["sm_scale"], topk_capacity=W)
    torch.cuda.synchronize()
    return out, lse


def test_writer_byte_exact_with_padding_rows():
    rng = np.random.default_rng(3)
    n, num_slots = 1000, 4096
    lat = wl.normal_bf16(rng, (n, 512))
    pe = wl.normal_bf16(rng, (n, 64))
    slots = rng.choice(np.arange(1, num_slots), size=n, replace=False).astype(np.int64)
    slots[-250:] = 0                                    # padding rows with NaN inputs, dropped
    lat[-250:] = 0x7FC0
    slots[5], slots[6] = -3, num_slots + 1
    for rope in (False, True):
        width = 576 if rope else 512
        cache = torch.full((num_slots, width), 3.0, dtype=torch.bfloat16, device=DEV)
        smla.kv_write_bf16(bf16_dev(lat), bf16_dev(pe) if rope else None, torch.from_numpy(slots).to(DEV), cache)
        torch.cuda.synchronize()
        host = np.full((num_slots, width), 0x4040, dtype=np.uint16)     # 3.0
        oracle_writer.kv_write_bf16(host, lat, pe if rope else None, slots)
        assert np.array_equal(_bits(cache), host)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_nope_decode_small_cache(T):
    print(f"bf16 nope decode T={T}", flush=True)
    cfg = wl.config_nope_decode(T, seed=400 + T, num_slots=16384, ctx=(512, 16384))
    cache = _build(cfg)
    out, lse = _run(cfg, cache, cfg["idx"])
    ref_out, ref_lse = _oracle(cfg, cache, cfg["idx"], range(T))
    assert_parity(out, lse, ref_out, ref_lse, range(T))


@pytest.mark.parametrize("T", [1, 16, 64])
def test_rope_decode_small_cache(T):
    """RoPE rows (512 + 64 bf16 values, 576-d scores), W = 2048."""
    print(f"bf16 rope decode T={T}", flush=True)
    cfg = wl.config_rope_decode(T, seed=430 + T, num_slots=32768, ctx=(2048, 30000))
    cache = _build(cfg)
    out, lse = _run(cfg, cache, cfg["idx"])
    ref_out, ref_lse = _oracle(cfg, cache, cfg["idx"], range(T))
    assert_parity(out, lse, ref_out, ref_lse, range(T))


@pytest.mark.parametrize("T", [65, 130])
def test_rope_prefill_rows(T):
    """Causal prefill rows over RoPE rows: row t lists tokens <= t, then -1."""
    print(f"bf16 rope prefill T={T}", flush=True)
    cfg = wl.config_prefill(T, num_slots=8192)
    cache = _build(cfg)
    out, lse = _run(cfg, cache, cfg["idx"])
    ref_out, ref_lse = _oracle(cfg, cache, cfg["idx"], range(T))
    assert_parity(out, lse, ref_out, ref_lse, range(T))


@pytest.mark.parametrize("rope", [False, True])
def test_padding_anywhere_empty_rows_and_out_of_range(rope):
    cfg = (wl.config_rope_decode(8, seed=411, num_slots=4096, ctx=(256, 4096), W=2176) if rope else
           wl.config_nope_decode(8, seed=410, num_slots=4096, ctx=(256, 4096)))
    cache = _build(cfg)
    rng = np.random.default_rng(7)
    idx = cfg["idx"].copy()
    for t in range(8):
        idx[t] = idx[t][rng.permutation(idx.shape[1])]   # padding scattered through the row
    idx[2] = -1                                          # a row with no valid entry
    idx[3, ::7] = cfg["num_slots"] + 5                   # out of range: padding
    idx[4, :3] = idx[4, 3]                               # duplicates count once each
    out, lse = _run(cfg, cache, idx)
    ref_out, ref_lse = _oracle(cfg, cache, idx, range(8))
    assert_parity(out, lse, ref_out, ref_lse, range(8))
    assert torch.all(out[2] == 0) and bool(torch.isneginf(lse[2]).all())


@pytest.mark.parametrize("H", [4, 16, 40])
@pytest.mark.parametrize("rope", [False, True])
def test_head_counts(H, rope):
    cfg = (wl.config_rope_decode(5, seed=425 + H, num_slots=4096, ctx=(256, 4096), H=H) if rope else
           wl.config_nope_decode(5, seed=420 + H, num_slots=4096, ctx=(256, 4096), H=H))
    cache = _build(cfg)
    out, lse = _run(cfg, cache, cfg["idx"])
    ref_out, ref_lse = _oracle(cfg, cache, cfg["idx"], range(5))
    assert_parity(out, lse, ref_out, ref_lse, range(5))


@pytest.mark.parametrize("rope", [False, True])
def test_full_size_decode_every_row(rope):
    """The full decode batches (T = 256: NoPE, 131,072-slot cache, W = 2176;
    RoPE, 262,144-slot cache, W = 2048), in the launch configuration the
    bench times; every row and head checked."""
    print(f"bf16 full decode rope={rope}", flush=True)
    cfg = wl.config_rope_decode(256) if rope else wl.config_nope_decode(256)
    cache = _build(cfg, check=False)
    out, lse = _run(cfg, cache, cfg["idx"])
    rows = list(range(256))
    ref_out, ref_lse = _oracle(cfg, cache, cfg["idx"], rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


@pytest.mark.parametrize("rope_dim", [0, 64])
def test_cache_beyond_4_gib(rope_dim):
    """4,500,000 rows of 1,024 or 1,152 bytes (4.6 / 5.2 GB): row byte offsets
    past 2^32 take the kernel's 64-bit address path."""
    num_slots = 4_500_000
    width = 512 + rope_dim
    assert num_slots * 2 * width > 2**32
    rng = np.random.default_rng(9 + rope_dim)
    cache = torch.zeros((num_slots, width), dtype=torch.bfloat16, device=DEV)
    T, W = 4, 512
    idx = np.stack([np.concatenate([rng.integers(4_200_000, num_slots, size=300),
                                    rng.integers(1, 1000, size=W - 300)]) for _ in range(T)]).astype(np.int32)
    uniq = np.unique(idx)
    lat = wl.normal_bf16(rng, (uniq.size, 512))
    pe = wl.normal_bf16(rng, (uniq.size, 64)) if rope_dim else None
    smla.kv_write_bf16(bf16_dev(lat), None if pe is None else bf16_dev(pe),
                       torch.from_numpy(uniq.astype(np.int64)).to(DEV), cache)
    q = wl.normal_bf16(rng, (T, 16, width))
    cfg = dict(num_slots=num_slots, q=q, sm_scale=float(1 / np.sqrt(width)))
    out, lse = _run(cfg, cache, idx)
    ref_out, ref_lse = _oracle(cfg, cache, idx, range(T))
    assert_parity(out, lse, ref_out, ref_lse, range(T))
