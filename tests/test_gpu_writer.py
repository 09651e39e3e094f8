"""HIP writer vs the oracle writer: byte-exact rows, dropped padding rows,
untouched bytes, NoPE zero tail, a sweep of every bf16 value and of every
reachable scale, and calls of random shape."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_fp8_amd as smla
import workloads as wl
from oracle import writer as oracle_writer
from tests.gpu_util import DEV, bf16_dev

pytestmark = pytest.mark.gpu


def _run(cfg, lat=None, rope=None):
    cache = torch.from_numpy(cfg["cache"]).to(DEV)
    lat_t = bf16_dev(cfg["latent"]) if lat is None else lat
    rope_t = (bf16_dev(cfg["rope"]) if cfg["rope"] is not None else None) if rope is None else rope
    smla.kv_write(lat_t, rope_t, torch.from_numpy(cfg["slots"]).to(DEV), cache)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


@pytest.mark.parametrize("N", [1024, 8192])
@pytest.mark.parametrize("rope_dim", [64, 0])
@pytest.mark.parametrize("shuffle", [False, True])
def test_writer_workload_byte_exact(N, rope_dim, shuffle):
    print(f"writer N={N} rope={rope_dim} shuffle={shuffle}", flush=True)
    cfg = wl.config_writer(N=N, rope_dim=rope_dim, shuffle=shuffle)
    got = _run(cfg)
    want = cfg["cache"].copy()
    keep = oracle_writer.kv_write(want, cfg["latent"], cfg["rope"], cfg["slots"])
    assert keep.sum() == N - N // 4
    assert not got[0].any(), "reserved slot 0 was written"
    if rope_dim == 0:
        assert not got[cfg["slots"][keep], 528:].any()
    assert np.array_equal(got, want)


def test_every_bf16_value_with_unit_scale():
    """Each tile holds 448 (so scale = 1 exactly and the quantiser input is x
    itself) plus 127 bf16 values; all finite bf16 values below 448 in
    magnitude are covered, which includes every e4m3 rounding tie."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    vals = bits[np.isfinite(x) & (np.abs(x) < 448.0)].astype(np.uint16)
    n_tiles = (vals.size + 126) // 127
    tiles = np.zeros((n_tiles, 128), dtype=np.uint16)
    flat = np.zeros(n_tiles * 127, dtype=np.uint16)
    flat[: vals.size] = vals
    tiles[:, 1:] = flat.reshape(n_tiles, 127)
    tiles[:, 0] = 0x43E0                                   # 448.0
    n_rows = (n_tiles + 3) // 4
    lat = np.zeros((n_rows * 4, 128), dtype=np.uint16)
    lat[:n_tiles] = tiles
    lat[n_tiles:, 0] = 0x43E0
    lat = lat.reshape(n_rows, 512)
    num_slots = n_rows + 1
    cfg = dict(cache=np.zeros((num_slots, 656), dtype=np.uint8), latent=lat, rope=None,
               slots=np.arange(1, num_slots, dtype=np.int64))
    got = _run(cfg)
    want = cfg["cache"].copy()
    oracle_writer.kv_write(want, lat, None, cfg["slots"])
    assert np.array_equal(got, want)


def test_scales_across_magnitudes_and_zero_tiles():
    rng = np.random.default_rng(8)
    n = 400
    x = rng.standard_normal((n, 512)).astype(np.float32)
    x *= np.exp2(rng.integers(-120, 120, size=(n, 1))).astype(np.float32)
    x[5, 128:256] = 0.0                      # an all-zero tile
    x[6, 0:128] = -0.0                       # an all negative-zero tile
    x[7, 256:384] = 0.0
    x[7, 300] = -1e-30                       # one tiny value in a zero tile
    lat = wl.bf16_bits_from_f32(x)
    rope = wl.normal_bf16(rng, (n, 64))
    cfg = dict(cache=np.full((n + 1, 656), 0x5A, dtype=np.uint8), latent=lat, rope=rope,
               slots=np.arange(1, n + 1, dtype=np.int64))
    got = _run(cfg)
    want = cfg["cache"].copy()
    oracle_writer.kv_write(want, lat, rope, cfg["slots"])
    assert np.array_equal(got, want)
    assert np.all(got[0] == 0x5A)


def test_strided_views_of_one_kv_tensor():
    """kv_c and k_pe as column slices of one [N][576] tensor (row stride 576)."""
    rng = np.random.default_rng(9)
    n, num_slots = 777, 5000
    full = wl.normal_bf16(rng, (n, 576))
    slots = rng.choice(num_slots - 1, size=n, replace=False).astype(np.int64) + 1
    slots[::10] = 0
    t = bf16_dev(full)
    cfg = dict(cache=np.zeros((num_slots, 656), dtype=np.uint8), latent=full[:, :512],
               rope=full[:, 512:], slots=slots)
    got = _run(cfg, lat=t[:, :512], rope=t[:, 512:])
    want = cfg["cache"].copy()
    oracle_writer.kv_write(want, full[:, :512], full[:, 512:], slots)
    assert np.array_equal(got, want)


def test_out_of_range_slots_are_dropped():
    rng = np.random.default_rng(10)
    num_slots = 100
    lat = wl.normal_bf16(rng, (6, 512))
    slots = np.array([-5, 0, 100, 1 << 40, 99, 1], dtype=np.int64)
    cfg = dict(cache=np.full((num_slots, 656), 0xA5, dtype=np.uint8), latent=lat, rope=None,
               slots=slots)
    cfg["cache"][0] = 0
    got = _run(cfg)
    want = cfg["cache"].copy()
    oracle_writer.kv_write(want, lat, None, slots)
    assert np.array_equal(got, want)


def _tiles_below(amax_bits: int) -> np.ndarray:
    """Tiles of 128 bf16 values: element 0 is the tile maximum (amax_bits, so
    every tile has the same scale) and the rest run through every bf16 value
    of smaller magnitude, both signs, and -amax."""
    bits = np.arange(1 << 15, dtype=np.uint32)
    vals = bits[bits < amax_bits]
    vals = np.concatenate([vals, vals | 0x8000, [amax_bits | 0x8000]]).astype(np.uint16)
    n_tiles = (vals.size + 126) // 127
    tiles = np.zeros((n_tiles, 128), dtype=np.uint16)
    flat = np.zeros(n_tiles * 127, dtype=np.uint16)
    flat[: vals.size] = vals
    tiles[:, 1:] = flat.reshape(n_tiles, 127)
    tiles[:, 0] = amax_bits
    return tiles


# Biased bf16 exponents of the tile maximum swept over all 128 mantissas.  A
# scale is fl32(amax / 448) with amax a bf16 value, so its mantissa takes only
# 128 values per exponent.  The kernel's reciprocal fast path serves scales
# >= 2^-60, i.e. amax >= 1.75 * 2^-52: exponent 75 (2^-52) straddles that
# threshold at mantissa 96, 76 lies above it and 74 below; 254 holds the
# largest finite maxima, 1 and 0 the smallest normal and the subnormal ones.
SWEEP_EXPONENTS = [127, 254, 76, 75, 74, 1, 0]


@pytest.mark.parametrize("amax_exp", SWEEP_EXPONENTS)
def test_every_reachable_scale_byte_exact(amax_exp):
    """Every tile maximum of one bf16 exponent (all 128 mantissas), each with
    every smaller bf16 magnitude of both signs: every quotient x / scale the
    writer can meet at these scales, its e4m3 rounding and every tie, is
    compared byte for byte with the oracle writer."""
    print(f"amax exponent {amax_exp}", flush=True)
    tiles = np.concatenate([_tiles_below((amax_exp << 7) | m) for m in range(128)
                            if (amax_exp, m) != (0, 0)])
    pad = (-tiles.shape[0]) % 4
    if pad:
        tiles = np.concatenate([tiles, tiles[:pad]])
    lat = tiles.reshape(-1, 512)
    n = lat.shape[0]
    cfg = dict(cache=np.zeros((n + 1, 656), dtype=np.uint8), latent=lat, rope=None,
               slots=np.arange(1, n + 1, dtype=np.int64))
    got = _run(cfg)
    want = cfg["cache"].copy()
    oracle_writer.kv_write(want, lat, None, cfg["slots"])
    assert np.array_equal(got, want)


def test_nan_input_in_a_kept_row():
    """A NaN in a kept row is not sanitised: its tile stores a NaN scale and NaN
    codes (0x7F or 0xFF) only, as the oracle's amax = NaN gives; the row's
    other tiles are exact."""
    rng = np.random.default_rng(12)
    lat = wl.normal_bf16(rng, (4, 512))
    lat[1, 200] = 0x7FC0                     # NaN in tile 1 of row 1
    lat[2, 5] = 0xFFC0                       # negative NaN in tile 0 of row 2
    cfg = dict(cache=np.zeros((5, 656), dtype=np.uint8), latent=lat, rope=None,
               slots=np.arange(1, 5, dtype=np.int64))
    got = _run(cfg)
    want = cfg["cache"].copy()
    oracle_writer.kv_write(want, lat, None, cfg["slots"])
    for row, tile in ((2, 1), (3, 0)):
        codes = got[row, 128 * tile:128 * (tile + 1)]
        assert np.all((codes & 0x7F) == 0x7F)
        assert np.isnan(got[row, 512 + 4 * tile:516 + 4 * tile].view("<f4")[0])
        assert np.all(np.isnan(oracle_writer.encode_rows(lat[row - 1:row], None)[0, 512:528]
                               .view("<f4")[tile:tile + 1]))
        keep = np.ones(656, dtype=bool)
        keep[128 * tile:128 * (tile + 1)] = False
        keep[512 + 4 * tile:516 + 4 * tile] = False
        assert np.array_equal(got[row][keep], want[row][keep])
    assert np.array_equal(got[[0, 1, 4]], want[[0, 1, 4]])


@pytest.mark.parametrize("seed", range(24))
def test_writer_random_calls(seed):
    """Writer calls of random shape, byte for byte against the oracle over the
    whole cache: ragged row counts, rope 0 or 64, inputs as column views of a
    wider tensor, rows scaled across binades with zero tiles, and padding rows
    (slot 0, negative, past the cache) holding NaN inputs; every byte the call
    must not write keeps its 0xA5 fill."""
    rng = np.random.default_rng(700 + seed)
    rope_dim = int(rng.choice([0, 64]))
    n = int(rng.choice([1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1000, 4097]))
    num_slots = int(rng.choice([300, 4096, 70000]))
    pad_cols = int(rng.choice([0, 64, 576]))
    print(f"writer sweep seed={seed} n={n} rope={rope_dim} slots={num_slots} pad={pad_cols}", flush=True)
    width = 512 + rope_dim + pad_cols
    x = wl.f32_from_bf16_bits(wl.normal_bf16(rng, (n, width)))
    x *= np.exp2(rng.integers(-60, 60, size=(n, 1))).astype(np.float32)
    zero_tile = rng.random((n, 4)) < 0.05
    for t in range(4):
        x[zero_tile[:, t], 128 * t:128 * (t + 1)] = 0.0
    full = wl.bf16_bits_from_f32(x.astype(np.float32))
    keep = min(n, num_slots - 1)
    slots = np.empty(n, dtype=np.int64)
    slots[:keep] = rng.choice(np.arange(1, num_slots), size=keep, replace=False)
    slots[keep:] = 0
    pad = rng.random(n) < 0.2
    slots[pad] = rng.choice([0, -1, -9, num_slots, num_slots + 77], size=int(pad.sum()))
    full[slots <= 0] = wl.BF16_QNAN
    full[slots >= num_slots] = wl.BF16_QNAN
    t_full = bf16_dev(full)
    lat_t = t_full[:, :512]
    rope_t = t_full[:, 512:512 + rope_dim] if rope_dim else None
    cache0 = np.full((num_slots, 656), 0xA5, dtype=np.uint8)
    cfg = dict(cache=cache0, latent=full[:, :512], rope=full[:, 512:512 + rope_dim] if rope_dim else None,
               slots=slots)
    got = _run(cfg, lat=lat_t, rope=rope_t)
    want = cache0.copy()
    oracle_writer.kv_write(want, full[:, :512], full[:, 512:512 + rope_dim] if rope_dim else None, slots)
    assert np.array_equal(got, want)
