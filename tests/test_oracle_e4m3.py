"""Pins of the oracle's E4M3 codec against the format definition and a library cast."""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codepoints.txt")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        out.append((int(c, 16), float(v)))
    return out


def test_codepoints_decode():
    for code, val in _golden():
        got = e4m3.decode(np.array([code], dtype=np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_codepoints_encode():
    for code, val in _golden():
        if np.isnan(val):
            continue
        assert int(e4m3.encode(np.array([val]))[0]) == code, hex(code)


def test_only_two_nan_codes():
    t = e4m3.decode_table()
    assert sorted(np.nonzero(np.isnan(t))[0].tolist()) == [0x7F, 0xFF]
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert codes.size == 254
    back = e4m3.encode(e4m3.decode(codes))
    assert np.array_equal(back, codes)


def test_midpoints_round_to_even():
    t = e4m3.decode_table()
    for c in range(0x00, 0x7E):            # adjacent positive codes c, c+1
        lo, hi = t[c], t[c + 1]
        mid = (lo + hi) / 2                # exact in f64 and in f32
        want = c if c % 2 == 0 else c + 1
        assert int(e4m3.encode(np.array([mid]))[0]) == want, hex(c)
        assert int(e4m3.encode(np.array([-mid]))[0]) == want | 0x80, hex(c)
        # just off the midpoint goes to the nearer code
        eps = (hi - lo) / 1024
        assert int(e4m3.encode(np.array([mid - eps]))[0]) == c
        assert int(e4m3.encode(np.array([mid + eps]))[0]) == c + 1


def test_saturation_and_signed_zero():
    v = np.array([448.0, 449.0, 463.0, 464.0, 479.0, 480.0, 1e6, 3.0e38,
                  -448.5, -1e30, -2.0 ** -11, -0.0, 2.0 ** -11, 0.0])
    want = [0x7E] * 8 + [0xFE, 0xFE, 0x80, 0x80, 0x00, 0x00]
    assert e4m3.encode(v).tolist() == want


def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_against_torch_cast_all_bf16_values():
    """Every finite bf16 value of magnitude < 464 (the whole rounding range of
    the format) encodes as torch's CPU float8_e4m3fn cast does."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x32 = (bits << 16).view(np.float32)
    ok = np.isfinite(x32) & (np.abs(x32) < 464.0)
    x32 = x32[ok]
    assert np.array_equal(e4m3.encode(x32.astype(np.float64)), _torch_e4m3(x32))


def test_against_torch_cast_random_f32():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000) * 100,
        rng.standard_normal(200000) * 0.01,          # subnormal region of e4m3
        rng.uniform(-463.9, 463.9, 200000),
    ]).astype(np.float32)
    assert np.array_equal(e4m3.encode(x.astype(np.float64)), _torch_e4m3(x))


@pytest.mark.parametrize("c", [0x01, 0x08, 0x38, 0x7E])
def test_neighbours_of_codes(c):
    """The float32 neighbours of a code value encode to that code."""
    v = np.float32(e4m3.decode_table()[c])
    for u in (np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(1000))):
        assert int(e4m3.encode(np.array([np.float64(u)]))[0]) == c
