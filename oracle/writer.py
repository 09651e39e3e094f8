"""Packing of MLA KV rows into the 656-byte fp8_ds_mla cache row.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Row layout (vLLM PR 55277, Purpose (1) and its Changes table): 512 bytes of
latent codes, 16 bytes of tile scales, 128 bytes of RoPE or padding = 656 B,
the same for NoPE models, whose 128-byte tail is written as zeros.  16 bytes
for the four 128-element tiles of the 512-wide latent means one 4-byte float32
scale per tile; the RoPE part is 64 bf16 values (128 bytes).

Writes aimed at the reserved padding slot 0 are dropped and their inputs are
never looked at (sglang PR 47013, Summary and Modifications: padding rows of a
batch point at the reserved slot, and what they carry is undefined).  Out-of-range
slots (< 0 or >= num_slots) are dropped as well; that part is this
implementation's reading, not something the pages state.

Steps, per kept row:
  W2  widen the bf16 inputs to float64 (exact);
  W3  per tile i: amax_i = max |x|, scale_i = fl32(amax_i / 448);
  W4  per element: v = fl32(x / scale_i), code = E4M3 RNE satfinite (v);
      a tile with amax_i == 0 stores scale 0 and all codes 0x00;
  W5  bytes [0,512) codes, [512,528) scales as little-endian float32,
      [528,656) the RoPE bf16 bits little-endian, or zeros when rope_dim == 0.
fl32(a / b) is computed as a float64 quotient rounded once to float32; with
53 >= 2*24 + 2 bits this double rounding equals IEEE float32 division
(Figueroa, "When is double rounding innocuous?", 1995).
"""
from __future__ import annotations

import numpy as np

from . import e4m3

ROW_BYTES = 656
LATENT = 512
TILE = 128
N_TILES = LATENT // TILE
SCALE_OFF = 512
ROPE_OFF = 528


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def _fl32(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def encode_rows(latent_bits: np.ndarray, rope_bits: np.ndarray | None) -> np.ndarray:
    """Packed 656-byte rows for every input row (no slot logic): uint8 [N][656]."""
    latent_bits = np.asarray(latent_bits, dtype=np.uint16)
    n = latent_bits.shape[0]
    x = _bf16_to_f64(latent_bits).reshape(n, N_TILES, TILE)            # W2
    amax = np.max(np.abs(x), axis=2)                                    # W3
    scale = _fl32(amax / 448.0)
    zero_tile = amax == 0.0
    safe = np.where(zero_tile, 1.0, scale)
    v = _fl32(x / safe[:, :, None])                                     # W4
    codes = e4m3.encode(v)
    codes[zero_tile] = 0x00
    rows = np.zeros((n, ROW_BYTES), dtype=np.uint8)                      # W5
    rows[:, :LATENT] = codes.reshape(n, LATENT)
    rows[:, SCALE_OFF:ROPE_OFF] = (
        scale.astype("<f4").view(np.uint8).reshape(n, 4 * N_TILES))
    if rope_bits is not None:
        rb = np.asarray(rope_bits, dtype=np.uint16)
        assert rb.shape == (n, 64), "rope part must be 64 bf16 values"
        rows[:, ROPE_OFF:] = rb.astype("<u2").view(np.uint8).reshape(n, 128)
    return rows


def kv_write(cache: np.ndarray, latent_bits: np.ndarray, rope_bits: np.ndarray | None,
             slots: np.ndarray) -> np.ndarray:
    """Write rows into `cache` (uint8 [num_slots][656]) in place; return the keep mask.

    W1: a row is kept iff 1 <= slot < num_slots; a dropped row's inputs are
    never read (its entries may hold NaN).  W6: no other byte changes."""
    num_slots = cache.shape[0]
    assert cache.shape[1] == ROW_BYTES and cache.dtype == np.uint8
    slots = np.asarray(slots, dtype=np.int64)
    keep = (slots >= 1) & (slots < num_slots)                           # W1
    kept = np.nonzero(keep)[0]
    if kept.size:
        rows = encode_rows(np.asarray(latent_bits)[kept],
                           None if rope_bits is None else np.asarray(rope_bits)[kept])
        cache[slots[kept]] = rows
    return keep


def kv_write_bf16(cache_bits: np.ndarray, latent_bits: np.ndarray, rope_bits: np.ndarray | None,
                  slots: np.ndarray) -> np.ndarray:
    """BF16 KV cache (sglang PR 47013, Speed Tests: rows of 512 bf16 values):
    cache_bits uint16 [num_slots][512 + rope_dim] receives each kept row's bf16
    values unchanged, in place; the slot rule W1 and W6 are those of the
    quantised cache.  Returns the keep mask."""
    num_slots, width = cache_bits.shape
    rope_dim = 0 if rope_bits is None else 64
    assert width == 512 + rope_dim and cache_bits.dtype == np.uint16
    slots = np.asarray(slots, dtype=np.int64)
    keep = (slots >= 1) & (slots < num_slots)
    kept = np.nonzero(keep)[0]
    if kept.size:
        row = np.asarray(latent_bits, dtype=np.uint16)[kept, :512]
        if rope_dim:
            row = np.concatenate([row, np.asarray(rope_bits, dtype=np.uint16)[kept, :64]], axis=1)
        cache_bits[slots[kept]] = row
    return keep


def unfiltered_kv_write(cache: np.ndarray, latent_bits: np.ndarray, rope_bits: np.ndarray | None,
                        slots: np.ndarray) -> np.ndarray:
    """NEGATIVE CONTROL ONLY: the zero-RoPE writer as it was before the fix of
    sglang PR 47013 (Summary and Motivation), which drops no write aimed at the
    reserved slot 0.  Every row with 0 <= slot < num_slots is packed and
    stored, so the padding rows of a batch (undefined inputs, NaN here) land in
    slot 0, the last of them winning.  Kept so that a test can show the slot-0
    check failing for it while kv_write above passes."""
    num_slots = cache.shape[0]
    slots = np.asarray(slots, dtype=np.int64)
    keep = (slots >= 0) & (slots < num_slots)
    for i in np.nonzero(keep)[0]:                  # in row order: the last row for a slot wins
        cache[slots[i]] = encode_rows(np.asarray(latent_bits)[i:i + 1],
                                      None if rope_bits is None else np.asarray(rope_bits)[i:i + 1])[0]
    return keep
