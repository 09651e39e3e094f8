"""Gather + upconvert of fp8_ds_mla cache rows into bf16 rows, reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (vLLM PR 55277, Purpose (1), and the review of its cache
gather for the chunked-context path: with pe_dim 0 the reader gets exact zeros
in columns 512..575 rather than stale cache bytes).  For each listed slot:

  G1  0 <= slot < num_slots selects the row (slot 0 included: it is a real,
      reserved slot); any other entry gives an all-zero output row.
  G2  value e < 512: E4M3(code[e]) * scale[e // 128], exact in float64 (4 + 24
      significant bits), rounded to float32 (nearest even), then to bf16
      (nearest even); NaN codes give the bf16 NaN 0x7FC0.
  G3  columns 512..575: the row's 64 bf16 RoPE values (rope_dim 64), or +0
      (rope_dim 0: the row's tail bytes are not looked at).

Reading: the pages name the gather but not the rounding; the dequantised
value is formed in the precision of the stored scale (float32) and cast to
bf16 once, which is what "upconvert" of an fp32-scaled value gives.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

ROW_BYTES = 656
LATENT = 512
TILE = 128
SCALE_OFF = 512
ROPE_OFF = 528
OUT_WIDTH = 576


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even; NaN -> 0x7FC0."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return np.where(nan, 0x7FC0, r).astype(np.uint16)


def gather_upconvert(cache: np.ndarray, slots: np.ndarray, rope_dim: int) -> np.ndarray:
    """cache uint8 [num_slots][656]; slots int64 [N] -> bf16 bits uint16 [N][576]."""
    slots = np.asarray(slots, dtype=np.int64)
    n = slots.shape[0]
    out = np.zeros((n, OUT_WIDTH), dtype=np.uint16)
    ok = (slots >= 0) & (slots < cache.shape[0])                        # G1
    if not ok.any():
        return out
    rows = cache[slots[ok]]
    codes = rows[:, :LATENT]
    scales = np.ascontiguousarray(rows[:, SCALE_OFF:ROPE_OFF]).view("<f4").astype(np.float64)
    with np.errstate(invalid="ignore"):
        v = e4m3.decode(codes).reshape(-1, 4, TILE) * scales[:, :, None]  # G2, exact
    out[ok, :LATENT] = f32_to_bf16_bits(v.reshape(-1, LATENT).astype(np.float32))
    if rope_dim:                                                         # G3
        out[ok, LATENT:] = np.ascontiguousarray(rows[:, ROPE_OFF:ROW_BYTES]).view("<u2")
    return out
