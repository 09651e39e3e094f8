"""Pins of the oracle's gather + upconvert: torch's own float8_e4m3fn decode,
float32 multiply and bfloat16 cast on the same bytes, closed forms at the
edges of the formats, the NoPE zero tail over sentinel bytes, and invalid
entries."""
import numpy as np
import torch

import workloads as wl
from oracle import gather as G
from oracle import writer


def _cache(num_slots, rope_dim, seed, tail=None):
    rng = np.random.default_rng(seed)
    lat, rope, slots = wl.cache_rows(rng, num_slots, rope_dim)
    lat = (wl.f32_from_bf16_bits(lat) * np.exp2(rng.integers(-30, 30, size=(lat.shape[0], 1)))).astype(np.float32)
    lat = wl.bf16_bits_from_f32(lat)
    cache = np.zeros((num_slots, 656), dtype=np.uint8)
    writer.kv_write(cache, lat, rope, slots)
    if tail is not None:
        cache[:, 528:] = tail
    cache[0] = wl.slot0_bytes(rng, "ff")
    return rng, cache


def _torch_upconvert(cache, slots, rope_dim):
    rows = torch.from_numpy(cache[np.asarray(slots)].copy())
    codes = rows[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
    sc = rows[:, 512:528].contiguous().view(torch.float32)
    v = (codes.view(-1, 4, 128) * sc[:, :, None]).reshape(-1, 512)   # float32 multiply
    out = torch.zeros((len(slots), 576), dtype=torch.bfloat16)
    out[:, :512] = v.to(torch.bfloat16)
    if rope_dim:
        out[:, 512:] = rows[:, 528:].contiguous().view(torch.bfloat16)
    return out.view(torch.int16).numpy().view(np.uint16)


def test_matches_torch_casts_rope_and_nope():
    for rope_dim, seed in ((64, 1), (0, 2)):
        rng, cache = _cache(2048, rope_dim, seed)
        slots = rng.choice(np.arange(1, 2048), size=700, replace=False)
        got = G.gather_upconvert(cache, slots, rope_dim)
        assert np.array_equal(got, _torch_upconvert(cache, slots, rope_dim))


def test_nope_tail_is_zero_whatever_the_cache_holds():
    rng, cache = _cache(512, 0, 3, tail=0xA5)
    got = G.gather_upconvert(cache, np.arange(1, 512), 0)
    assert np.all(got[:, 512:] == 0)
    # and the RoPE layout copies the tail bit for bit
    got64 = G.gather_upconvert(cache, np.arange(1, 512), 64)
    assert np.all(got64[:, 512:] == 0xA5A5)


def test_invalid_entries_give_zero_rows_and_slot0_is_read():
    rng, cache = _cache(256, 64, 4)
    slots = np.array([-1, 5, 256, 1 << 40, 0, -7])
    got = G.gather_upconvert(cache, slots, 64)
    assert np.all(got[[0, 2, 3, 5]] == 0)
    assert np.array_equal(got[1], G.gather_upconvert(cache, np.array([5]), 64)[0])
    # slot 0 holds 0xFF bytes: NaN codes -> 0x7FC0, and its tail copied as is
    assert np.all(got[4, :512] == 0x7FC0) and np.all(got[4, 512:] == 0xFFFF)


def test_closed_forms():
    cache = np.zeros((2, 656), dtype=np.uint8)
    cache[1, 0] = 0x38                    # 1.0
    cache[1, 1] = 0xB8                    # -1.0
    cache[1, 2] = 0x7E                    # 448
    cache[1, 3] = 0x01                    # 2^-9
    cache[1, 4] = 0x80                    # -0
    cache[1, 128] = 0x38
    cache[1, 512:516] = np.frombuffer(np.float32(0.5).tobytes(), np.uint8)
    cache[1, 516:520] = np.frombuffer(np.float32(2.0**-120).tobytes(), np.uint8)
    got = G.gather_upconvert(cache, np.array([1]), 0)[0]
    assert got[0] == 0x3F00               # 0.5
    assert got[1] == 0xBF00               # -0.5
    assert got[2] == 0x4360               # 224
    assert got[3] == 0x3A80               # 2^-10
    assert got[4] == 0x8000               # -0 keeps its sign
    assert got[5] == 0x0000
    assert got[128] == 0x0380             # 2^-120 (a normal bf16: exponent 7, mantissa 0)
    # the rounding goes through float32: 1.125 * s with s = 0x1.c8e39p-1 is
    # exactly (1 + 2^-8) + 2^-24, half a float32 ulp above the bf16 tie
    # 1 + 2^-8; float32 rounds it onto the tie (to even), bf16 then to even
    # (0x3F80), whereas one rounding of the exact product would give 0x3F81
    c2 = np.zeros((1, 656), dtype=np.uint8)
    c2[0, 0] = 0x39                       # 1.125
    s = np.float32(float.fromhex("0x1.c8e39p-1"))
    assert 1.125 * float(s) == 1 + 2.0**-8 + 2.0**-24
    c2[0, 512:516] = np.frombuffer(s.tobytes(), np.uint8)
    assert G.gather_upconvert(c2, np.array([0]), 0)[0, 0] == 0x3F80
    assert _torch_upconvert(c2, [0], 0)[0, 0] == 0x3F80
