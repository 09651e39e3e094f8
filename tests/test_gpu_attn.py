"""HIP sparse attention vs the float64 oracle on the same cache bytes:
poisoned slot 0, NoPE and RoPE decode, prefill across the 64/65 boundary,
the widened top-k buffer, permutations, empty rows and head counts."""
import functools

import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from tests.gpu_util import DEV, assert_parity, bf16_dev, build_cache, oracle_for, run_attn

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _tiny():
    return wl.config_tiny()


@pytest.mark.parametrize("poison", ["ff", "7f", "random", "zero"])
def test_tiny_poisoned_slot0(poison):
    print(f"tiny poison={poison}", flush=True)
    cfg = dict(_tiny())
    cfg["slot0"] = wl.slot0_bytes(np.random.default_rng(3), poison)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    ref_out, ref_lse = oracle_for(cfg, range(cfg["T"]))
    assert_parity(out, lse, ref_out, ref_lse, range(cfg["T"]))
    # identical bits whatever slot 0 holds
    cfg0 = dict(cfg)
    cfg0["slot0"] = wl.slot0_bytes(None, "zero")
    cache0 = build_cache(cfg0)
    out0, lse0 = run_attn(cfg0, cache0)
    assert torch.equal(out, out0) and torch.equal(lse, lse0)


def test_tiny_unreferenced_slots_do_not_matter():
    cfg = _tiny()
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    used = np.unique(cfg["idx"][cfg["idx"] >= 0])
    unused = np.setdiff1d(np.arange(cfg["num_slots"]), used)
    cache[torch.from_numpy(unused).to(DEV)] = 0xFF
    out2, lse2 = run_attn(cfg, cache)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_nope_decode_small_cache(T):
    """GLM-style NoPE decode (512-d scores, W = 2176 with a 128-wide -1 tail)
    on a 16,384-slot cache with contexts of 512..16k tokens."""
    print(f"nope decode T={T}", flush=True)
    cfg = wl.config_nope_decode(T, seed=100 + T, num_slots=16384, ctx=(512, 16384))
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    rows = range(T)
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_rope_decode_small_cache(T):
    print(f"rope decode T={T}", flush=True)
    cfg = wl.config_rope_decode(T, seed=200 + T, num_slots=32768, ctx=(2048, 32768))
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    rows = range(T)
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


@functools.lru_cache(maxsize=None)
def _full(kind):
    if kind == "nope":
        return wl.config_nope_decode(256)
    if kind == "rope":
        return wl.config_rope_decode(256)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["nope", "rope"])
def test_full_size_decode_every_row(kind):
    """The full decode workloads at 256 tokens (131,072 / 262,144 slots), in
    the launch configuration the benchmark times, every row and head checked.
    The oracle attends over the cache bytes the HIP writer produced, after
    4,096 of the referenced rows (and slot 0) are checked byte for byte against
    the oracle writer."""
    from oracle import attention as oracle_attn
    print(f"full decode {kind}", flush=True)
    cfg = _full(kind)
    rng = np.random.default_rng(5)
    need = np.unique(cfg["idx"][cfg["idx"] >= 0])
    cache = build_cache(cfg, check_slots=rng.choice(need, size=4096, replace=False))
    out, lse = run_attn(cfg, cache)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    host = cache.cpu().numpy()
    assert np.array_equal(host[0], cfg["slot0"])
    ref_out, ref_lse = oracle_attn.sparse_mla_attn(cfg["q"], host, cfg["idx"], cfg["idx"].shape[1],
                                                   cfg["rope_dim"], cfg["sm_scale"])
    assert_parity(out, lse, ref_out, ref_lse, range(cfg["T"]))


@pytest.mark.parametrize("rope_dim", [0, 64])
def test_disjoint_t256_every_row(rope_dim):
    """The no-reuse controls the benchmark times: 256 decode tokens whose
    top-k sets are pairwise disjoint on a 1,048,576-slot cache (NoPE in the
    2176-wide buffer, RoPE in a 2048-wide one), every row and head checked
    against the oracle on the cache bytes the HIP writer produced."""
    from oracle import attention as oracle_attn
    print(f"disjoint T=256 rope={rope_dim}", flush=True)
    cfg = wl.config_disjoint_t256(rope_dim)
    rng = np.random.default_rng(6)
    cache = build_cache(cfg, check_slots=rng.choice(cfg["slots"], size=4096, replace=False))
    out, lse = run_attn(cfg, cache)
    host = cache.cpu().numpy()
    del cache
    ref_out, ref_lse = oracle_attn.sparse_mla_attn(cfg["q"], host, cfg["idx"], cfg["idx"].shape[1],
                                                   cfg["rope_dim"], cfg["sm_scale"])
    assert_parity(out, lse, ref_out, ref_lse, range(cfg["T"]))


@pytest.mark.parametrize("T", [63, 64, 65, 66, 128])
def test_prefill_across_boundary(T):
    """Causal prefill rows (row t lists tokens <= t, then -1)."""
    print(f"prefill T={T}", flush=True)
    cfg = wl.config_prefill(T, num_slots=8192)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    rows = range(T)
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_prefill_1024_every_row():
    """Sparse prefill of one causal sequence of 1,024 rows (rope 64, W = 2048),
    in the launch configuration the benchmark times; every row and head is
    checked against the oracle run on the cache bytes the HIP writer produced
    (all 1,024 referenced rows checked byte for byte first)."""
    from oracle import attention as oracle_attn
    cfg = wl.config_prefill(1024)
    need = np.unique(cfg["idx"][cfg["idx"] >= 0])
    cache = build_cache(cfg, check_slots=need)
    out, lse = run_attn(cfg, cache)
    assert torch.isfinite(out.float()).all()
    host = cache.cpu().numpy()
    ref_out, ref_lse = oracle_attn.sparse_mla_attn(cfg["q"], host, cfg["idx"], cfg["idx"].shape[1],
                                                   cfg["rope_dim"], cfg["sm_scale"])
    assert_parity(out, lse, ref_out, ref_lse, range(cfg["T"]))


def test_row_boundary_64_65_consistent():
    """The first 64 rows come out the same whether the call has 64 or 65 rows."""
    cfg = wl.config_prefill(65, num_slots=8192)
    cache = build_cache(cfg)
    out65, lse65 = run_attn(cfg, cache)
    c64 = dict(cfg)
    c64["q"], c64["idx"] = cfg["q"][:64], cfg["idx"][:64]
    out64, lse64 = run_attn(c64, cache)
    d = (out65[:64].float() - out64.float()).abs().max().item()
    assert d <= 2e-2
    assert (lse65[:64] - lse64).abs().max().item() <= 1e-3


def test_permutation_and_capacity():
    """Shuffling a row (moving -1 into the middle), widening the buffer with a
    -1 tail, and junk entries past the capacity all leave the result in bounds."""
    cfg = wl.config_rope_decode(16, seed=300, num_slots=16384, ctx=(600, 4000))
    cache = build_cache(cfg)
    rows = range(16)
    ref_out, ref_lse = oracle_for(cfg, rows)
    rng = np.random.default_rng(1)
    shuf = np.stack([rng.permutation(r) for r in cfg["idx"]])
    out, lse = run_attn(cfg, cache, idx=shuf)
    assert_parity(out, lse, ref_out, ref_lse, rows)
    wide = np.full((16, 2176 + 40), 7, dtype=np.int32)    # junk past the capacity
    wide[:, :2048] = cfg["idx"]
    wide[:, 2048:2176] = -1
    out, lse = run_attn(cfg, cache, idx=wide, W=2176)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_empty_rows_duplicates_and_out_of_range():
    cfg = dict(_tiny())
    idx = cfg["idx"].copy()
    idx[0, :] = -1                          # no valid entry
    idx[1, 77:90] = idx[1, 0]               # duplicates of one entry
    idx[1, 90:95] = cfg["num_slots"] + 3    # out of range = padding
    idx[1, 95:100] = -7
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache, idx=idx)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ref_out, ref_lse = oracle_for(cfg, [0, 1], idx=idx)
    assert_parity(out, lse, ref_out, ref_lse, [0, 1])


@pytest.mark.parametrize("H", [1, 4, 20, 32, 128])
def test_head_counts(H):
    print(f"heads H={H}", flush=True)
    cfg = wl.config_rope_decode(3, seed=400 + H, num_slots=8192, ctx=(100, 3000), H=H)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    ref_out, ref_lse = oracle_for(cfg, range(3))
    assert_parity(out, lse, ref_out, ref_lse, range(3))


def test_deterministic():
    cfg = wl.config_nope_decode(16, seed=500, num_slots=16384, ctx=(512, 16384))
    cache = build_cache(cfg)
    a = run_attn(cfg, cache)
    b = run_attn(cfg, cache)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("rope_dim", [0, 64])
def test_cache_beyond_4_gib(rope_dim):
    """A cache of 7,000,000 slots (4.6 GB): row byte offsets past 2^32 take the
    kernel's 64-bit address path.  Only the referenced rows are written (on the
    GPU by the writer, and in the oracle's lazily zeroed host copy)."""
    from oracle import attention as oracle_attn
    from oracle import writer as oracle_writer
    print(f"cache beyond 4 GiB rope={rope_dim}", flush=True)
    num_slots = 7_000_000
    assert num_slots * wl.ROW_BYTES > 2**32
    rng = np.random.default_rng(600 + rope_dim)
    T, H, W = 4, 16, 384
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = 200 + 40 * t
        hi = rng.choice(np.arange(6_600_000, num_slots), size=n // 2, replace=False)   # beyond 4 GiB
        lo = rng.choice(np.arange(1, 6_500_000), size=n - n // 2, replace=False)
        v = np.concatenate([hi, lo])
        rng.shuffle(v)
        idx[t, :n] = v
    slots = np.unique(idx[idx >= 0]).astype(np.int64)
    latent = wl.normal_bf16(rng, (slots.size, 512))
    rope = wl.normal_bf16(rng, (slots.size, rope_dim)) if rope_dim else None
    cache = torch.empty((num_slots, wl.ROW_BYTES), dtype=torch.uint8, device=DEV)
    cache[0] = 0x7F
    lat_d = torch.from_numpy(latent.view(np.int16)).view(torch.bfloat16).to(DEV)
    rope_d = torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).to(DEV) if rope_dim else None
    smla.kv_write(lat_d, rope_d, torch.from_numpy(slots).to(DEV), cache)
    q = wl.normal_bf16(rng, (T, H, 512 + rope_dim))
    sm = float(1.0 / np.sqrt(512 + rope_dim))
    out, lse = smla.attn(torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(DEV), cache,
                         torch.from_numpy(idx).to(DEV), sm, rope_dim)
    torch.cuda.synchronize()
    host = np.zeros((num_slots, wl.ROW_BYTES), dtype=np.uint8)       # untouched pages stay unallocated
    host[slots] = oracle_writer.encode_rows(latent, rope)
    host[0] = 0x7F
    assert np.array_equal(cache[torch.from_numpy(slots).to(DEV)].cpu().numpy(), host[slots])
    ref_out, ref_lse = oracle_attn.sparse_mla_attn(q, host, idx, W, rope_dim, sm)
    del cache
    assert_parity(out, lse, ref_out, ref_lse, range(T))


# The largest cache the 32-bit gather path takes (its scalar base sits 4 KiB
# below the cache and 8 KiB of offset range stay free); one slot more takes the
# 64-bit path.
LARGEST_32BIT_SLOTS = (0xFFFFFFFF - 8192) // wl.ROW_BYTES


@pytest.mark.parametrize("T", [4, 300])
@pytest.mark.parametrize("rope_dim", [0, 64])
def test_largest_32bit_cache_and_lowest_slots(rope_dim, T):
    """The last slots of the largest cache the 32-bit gather path takes, and
    slots 1..6 (row offsets below the 4 KiB that the loads' instruction
    offsets reach), in every row; 4 rows run eight-wavefront workgroups, 300
    rows four-wavefront ones."""
    from oracle import attention as oracle_attn
    from oracle import writer as oracle_writer
    print(f"largest 32-bit cache rope={rope_dim} T={T}", flush=True)
    num_slots = LARGEST_32BIT_SLOTS
    assert (num_slots + 1) * wl.ROW_BYTES > 0xFFFFFFFF - 8192
    rng = np.random.default_rng(860 + rope_dim + T)
    H, W = 16, 160
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = 6 + 1 + (t * 37) % (W - 7)
        v = np.concatenate([np.arange(1, 7), [num_slots - 1],
                            rng.choice(np.arange(num_slots - 4000, num_slots - 1), size=n - 7, replace=False)])
        rng.shuffle(v)
        idx[t, :n] = v
    slots = np.unique(idx[idx >= 0]).astype(np.int64)
    latent = wl.normal_bf16(rng, (slots.size, 512))
    rope = wl.normal_bf16(rng, (slots.size, rope_dim)) if rope_dim else None
    cache = torch.empty((num_slots, wl.ROW_BYTES), dtype=torch.uint8, device=DEV)
    cache[0] = 0x7F
    lat_d = torch.from_numpy(latent.view(np.int16)).view(torch.bfloat16).to(DEV)
    rope_d = torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).to(DEV) if rope_dim else None
    smla.kv_write(lat_d, rope_d, torch.from_numpy(slots).to(DEV), cache)
    q = wl.normal_bf16(rng, (T, H, 512 + rope_dim))
    sm = float(1.0 / np.sqrt(512 + rope_dim))
    out, lse = smla.attn(torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(DEV), cache,
                         torch.from_numpy(idx).to(DEV), sm, rope_dim)
    torch.cuda.synchronize()
    host = np.zeros((num_slots, wl.ROW_BYTES), dtype=np.uint8)
    host[slots] = oracle_writer.encode_rows(latent, rope)
    host[0] = 0x7F
    ref_out, ref_lse = oracle_attn.sparse_mla_attn(q, host, idx, W, rope_dim, sm)
    del cache
    assert_parity(out, lse, ref_out, ref_lse, range(T))


def test_buffer_wider_than_one_scan():
    """A top-k buffer wider than one split's scan (3,000 > 2,304 entries): the
    row is cut into fixed ranges instead of dealt out; valid entries and -1
    padding interleaved across the whole width."""
    cfg = wl.config_rope_decode(2, seed=700, num_slots=16384, ctx=(4000, 16000), W=3000)
    rng = np.random.default_rng(7)
    idx = np.full((2, 3000), -1, dtype=np.int32)
    for t in range(2):
        n = 2500 - 700 * t
        pos = np.sort(rng.choice(3000, size=n, replace=False))
        idx[t, pos] = rng.choice(np.arange(1, 16384), size=n, replace=False)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache, idx=idx)
    ref_out, ref_lse = oracle_for(cfg, [0, 1], idx=idx)
    assert_parity(out, lse, ref_out, ref_lse, [0, 1])


def test_maximum_row_count():
    """65,535 query rows (the largest call): one workgroup per row; sampled
    rows against the oracle, every row finite."""
    print("max rows", flush=True)
    base = _tiny()
    rng = np.random.default_rng(21)
    T, W = 65535, 8
    idx = np.full((T, W), -1, dtype=np.int32)
    idx[:, :5] = rng.integers(1, base["num_slots"], size=(T, 5))
    cfg = dict(base, T=T, H=1, W=W, q=wl.normal_bf16(rng, (T, 1, 576)), idx=idx)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = np.concatenate([np.arange(0, 64), rng.choice(T, size=64, replace=False), np.arange(T - 64, T)])
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


@pytest.mark.parametrize("T,poison", [(65, "ff"), (65, "7f"), (64, "ff"), (64, "random")])
def test_page_harness_shapes_have_no_nan_rows(T, poison):
    """The kernel-harness shapes of sglang PR 39288, Root cause (one 64-page
    cache, H = 16, T = 65 prefill / 64 decode rows, most of them padded with
    -1, slot 0 holding NaN-coded or random bytes): where a reader that clamps
    -1 to slot 0 turns every padded row into NaN, this kernel gives no NaN
    and matches the oracle, bit for bit the same output as with slot 0 zeroed."""
    print(f"harness T={T} slot0={poison}", flush=True)
    rng = np.random.default_rng(900 + T)
    num_slots, W = 64 * 64, 44 if T == 65 else 43
    latent, rope, slots = wl.cache_rows(rng, num_slots, 64)
    idx, _ = wl.prefill_topk(rng, T, W, num_slots)
    assert int((idx < 0).any(axis=1).sum()) >= W - 1
    cfg = dict(num_slots=num_slots, rope_dim=64, T=T, H=16, W=W, latent=latent, rope=rope,
               slots=slots, q=wl.normal_bf16(rng, (T, 16, 576)), idx=idx,
               sm_scale=float(1 / np.sqrt(576)), slot0=wl.slot0_bytes(rng, poison))
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ref_out, ref_lse = oracle_for(cfg, range(T))
    assert_parity(out, lse, ref_out, ref_lse, range(T))
    cache[0] = 0
    out0, lse0 = run_attn(cfg, cache)
    assert torch.equal(out, out0) and torch.equal(lse, lse0)


def test_single_entry_rows_and_an_all_padding_batch():
    """Degenerate lists: width 1 (a row attends to one key, so its output is
    that key's dequantised latent and its LSE that key's score; a -1 there
    leaves the row empty), and a batch whose every entry is padding."""
    cfg = dict(_tiny())
    rng = np.random.default_rng(23)
    T = 6
    idx = rng.integers(1, cfg["num_slots"], size=(T, 1)).astype(np.int32)
    idx[2, 0] = -1
    cfg.update(T=T, H=4, W=1, idx=idx, q=wl.normal_bf16(rng, (T, 4, 576)))
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    ref_out, ref_lse = oracle_for(cfg, range(T))
    assert_parity(out, lse, ref_out, ref_lse, range(T))
    assert torch.all(out[2] == 0) and bool(torch.isneginf(lse[2]).all())
    pad = np.full((T, 300), -1, dtype=np.int32)
    out, lse = run_attn(cfg, cache, idx=pad)
    assert torch.all(out == 0) and bool(torch.isneginf(lse).all())


# ---- calls with more (row, head group) units than one round of eight-wavefront
# workgroups run four-wavefront workgroups (32-key chunks, two per CU)

@pytest.mark.parametrize("kind,T,H", [("nope", 300, 16), ("rope", 260, 32), ("rope", 257, 16),
                                        ("nope", 140, 20)])
def test_four_wave_decode_every_row(kind, T, H):
    print(f"four-wave {kind} T={T} H={H}", flush=True)
    if kind == "nope":
        cfg = wl.config_nope_decode(T, seed=800 + T, num_slots=16384, ctx=(512, 16000), H=H)
    else:
        cfg = wl.config_rope_decode(T, seed=800 + T, num_slots=32768, ctx=(2048, 32000), H=H)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    rows = range(T)
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_four_wave_chunk_edges_and_empty_rows():
    """Rows of 0, 1, 31, 32, 33, 63, 64, 65 and more entries, padding spread
    through the buffer, in a 300-row call (four-wavefront workgroups)."""
    cfg = wl.config_rope_decode(300, seed=810, num_slots=16384, ctx=(600, 12000))
    rng = np.random.default_rng(11)
    idx = np.full((300, 2048), -1, dtype=np.int32)
    counts = [0, 1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 2048]
    for t in range(300):
        n = counts[t % len(counts)] if t < 120 else int(rng.integers(0, 2049))
        pos = rng.choice(2048, size=n, replace=False)
        idx[t, pos] = rng.choice(np.arange(1, 16384), size=n, replace=False)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache, idx=idx)
    empty = np.nonzero((idx < 0).all(axis=1))[0]
    assert empty.size > 0
    assert torch.all(out[torch.from_numpy(empty).to(DEV)] == 0)
    rows = range(300)
    ref_out, ref_lse = oracle_for(cfg, rows, idx=idx)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_four_wave_buffer_wider_than_one_scan():
    """300 rows of a 3,000-wide buffer: fixed ranges of whole chunks (two splits
    per row, merged), four-wavefront workgroups."""
    cfg = wl.config_nope_decode(300, seed=820, num_slots=16384, ctx=(4000, 16000), W=3000)
    rng = np.random.default_rng(12)
    idx = np.full((300, 3000), -1, dtype=np.int32)
    for t in range(300):
        n = int(rng.integers(1, 2900))
        pos = np.sort(rng.choice(3000, size=n, replace=False))
        idx[t, pos] = rng.choice(np.arange(1, 16384), size=n, replace=False)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache, idx=idx)
    rows = range(300)
    ref_out, ref_lse = oracle_for(cfg, rows, idx=idx)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_eight_and_four_wave_workgroups_agree():
    """The first 256 rows of a 300-row call (four-wavefront workgroups) against
    the same 256 rows alone (eight-wavefront workgroups, one per row)."""
    cfg = wl.config_nope_decode(300, seed=830, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    out300, lse300 = run_attn(cfg, cache)
    c256 = dict(cfg)
    c256["q"], c256["idx"] = cfg["q"][:256], cfg["idx"][:256]
    out256, lse256 = run_attn(c256, cache)
    assert (out300[:256].float() - out256.float()).abs().max().item() <= 2e-2
    assert (lse300[:256] - lse256).abs().max().item() <= 1e-3


@pytest.mark.parametrize("rope_dim", [0, 64])
def test_four_wave_cache_beyond_4_gib(rope_dim):
    """300 rows over a 7,000,000-slot cache (4.6 GB): the four-wavefront
    kernel's 64-bit address path."""
    from oracle import attention as oracle_attn
    from oracle import writer as oracle_writer
    print(f"four-wave cache beyond 4 GiB rope={rope_dim}", flush=True)
    num_slots = 7_000_000
    rng = np.random.default_rng(840 + rope_dim)
    T, H, W = 300, 16, 96
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = 1 + t % W
        v = rng.choice(num_slots - 6_600_000, size=n, replace=False) + 6_600_000      # beyond 4 GiB
        v[: n // 2] = rng.choice(6_500_000 - 1, size=n // 2, replace=False) + 1
        idx[t, :n] = v
    slots = np.unique(idx[idx >= 0]).astype(np.int64)
    latent = wl.normal_bf16(rng, (slots.size, 512))
    rope = wl.normal_bf16(rng, (slots.size, rope_dim)) if rope_dim else None
    cache = torch.empty((num_slots, wl.ROW_BYTES), dtype=torch.uint8, device=DEV)
    cache[0] = 0x7F
    lat_d = torch.from_numpy(latent.view(np.int16)).view(torch.bfloat16).to(DEV)
    rope_d = torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16).to(DEV) if rope_dim else None
    smla.kv_write(lat_d, rope_d, torch.from_numpy(slots).to(DEV), cache)
    q = wl.normal_bf16(rng, (T, H, 512 + rope_dim))
    sm = float(1.0 / np.sqrt(512 + rope_dim))
    out, lse = smla.attn(torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(DEV), cache,
                         torch.from_numpy(idx).to(DEV), sm, rope_dim)
    torch.cuda.synchronize()
    host = np.zeros((num_slots, wl.ROW_BYTES), dtype=np.uint8)
    host[slots] = oracle_writer.encode_rows(latent, rope)
    host[0] = 0x7F
    ref_out, ref_lse = oracle_attn.sparse_mla_attn(q, host, idx, W, rope_dim, sm)
    del cache
    assert_parity(out, lse, ref_out, ref_lse, range(T))


# ---- two or three splits per row (eight-wavefront workgroups): the split of a
# row that finishes last merges the row inside the main launch

def _splits(T, H):
    return min(256 // (T * ((H + 15) // 16)), 34)


@pytest.mark.parametrize("kind,T,H", [("nope", 100, 16), ("rope", 90, 16), ("nope", 40, 32),
                                        ("rope", 70, 16), ("nope", 85, 3)])
def test_fused_merge_every_row(kind, T, H):
    print(f"fused merge {kind} T={T} H={H}", flush=True)
    assert 2 <= _splits(T, H) <= 3
    if kind == "nope":
        cfg = wl.config_nope_decode(T, seed=840 + T, num_slots=16384, ctx=(512, 16000), H=H)
    else:
        cfg = wl.config_rope_decode(T, seed=840 + T, num_slots=32768, ctx=(2048, 32000), H=H)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache)
    rows = range(T)
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_fused_merge_empty_and_short_rows():
    """100 rows (two splits each) of 0, 1, 2, 63..65, 127..129 and random
    entry counts with padding spread through the buffer: a split with no entry
    adds nothing to the merge, and a row with none gives zeros and -inf."""
    cfg = wl.config_nope_decode(100, seed=850, num_slots=16384, ctx=(600, 12000))
    rng = np.random.default_rng(13)
    W = cfg["W"]
    idx = np.full((100, W), -1, dtype=np.int32)
    counts = [0, 1, 2, 63, 64, 65, 127, 128, 129, 2048]
    for t in range(100):
        n = counts[t % len(counts)] if t < 40 else int(rng.integers(0, W + 1))
        pos = rng.choice(W, size=n, replace=False)
        idx[t, pos] = rng.choice(np.arange(1, 16384), size=n, replace=False)
    cache = build_cache(cfg)
    out, lse = run_attn(cfg, cache, idx=idx)
    empty = np.nonzero((idx < 0).all(axis=1))[0]
    assert empty.size > 0
    assert torch.all(out[torch.from_numpy(empty).to(DEV)] == 0)
    assert torch.all(torch.isneginf(lse[torch.from_numpy(empty).to(DEV)]))
    rows = range(100)
    ref_out, ref_lse = oracle_for(cfg, rows, idx=idx)
    assert_parity(out, lse, ref_out, ref_lse, rows)


def test_fused_merge_bits_do_not_depend_on_the_last_split():
    """Which split of a row arrives last varies from call to call (here also
    through the arrival words' starting contents, which add a retry to some
    arrivals); the merged bits must not.  These 100 rows (two splits each)
    hold an output within a rounding step of a bf16 tie (row 25, head 1, dim
    371), so a merge that weighs the last split by its own lane's copy of l,
    which can differ in its last bits from the stored one, flips it."""
    cfg = wl.config_nope_decode(300, seed=870, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    T = 100
    assert _splits(T, 16) == 2
    q = bf16_dev(cfg["q"][:T])
    idx = torch.from_numpy(np.ascontiguousarray(cfg["idx"][:T])).to(DEV)
    need = smla.workspace_size(T, 16, cfg["W"], 0)
    ref = None
    for i in range(24):
        if i % 3 == 0:
            ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
        elif i % 3 == 1:
            ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        o, l = smla.attn(q, cache, idx, cfg["sm_scale"], 0, workspace=ws)
        torch.cuda.synchronize()
        if ref is None:
            ref = (o, l)
        else:
            assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), i


def test_fused_merge_workspace_contents_do_not_matter():
    """The arrival words may start in any state: workspaces of random bytes,
    of 0xFF and of zeros, each shared by calls of other sizes in turn (a
    16-split call's partials land where the fused calls' words were), give the
    bits of a call on a fresh workspace every time."""
    cfg = wl.config_nope_decode(100, seed=860, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(DEV)
    sizes = (100, 70, 16, 85)
    assert [_splits(T, 16) for T in sizes] == [2, 3, 16, 3]
    ref = {T: smla.attn(q[:T].contiguous(), cache, idx[:T], cfg["sm_scale"], 0) for T in sizes}
    need = max(smla.workspace_size(T, 16, cfg["W"], 0) for T in sizes)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(14)
    for fill in ("random", "ff", "zero"):
        if fill == "random":
            ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=gen)
        else:
            ws = torch.full((need,), 0xFF if fill == "ff" else 0, dtype=torch.uint8, device=DEV)
        for T in sizes + sizes:
            o, l = smla.attn(q[:T].contiguous(), cache, idx[:T], cfg["sm_scale"], 0, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o, ref[T][0]) and torch.equal(l, ref[T][1]), (fill, T)
