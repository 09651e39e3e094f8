"""Sparse MLA attention over the fp8_ds_mla cache, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed (the plain definition; sglang PR 47013 Motivation, sglang PR
39288 Root cause (1), vLLM PR 55277 Purpose):

  A1  For query row t the valid entries are idx[t][k], k < W, with
      0 <= idx < num_slots; any negative entry (the pages use -1) is padding,
      wherever it sits in the row.  W is the buffer's capacity (vLLM PR 55277,
      Purpose (2): the width passed in is that of the physical buffer, and the
      -1 entries, not a length argument, mark where it is unused).  Duplicated
      entries count once each.
  A2  Each referenced row is dequantised: K[e] = E4M3(code[e]) * scale[e // 128]
      for e < 512, and K[512 + r] = bf16 RoPE value r when rope_dim = 64.
  A3  s_j = sm_scale * sum_d q[t,h,d] * K_j[d] over d < 512 + rope_dim.
  A4  p_j = exp(s_j - m) / sum exp(s_j - m), m = max s_j.
  A5  o[t,h] = sum_j p_j * K_j[0:512] (the latent is the value), and
      lse[t,h] = m + ln sum exp(s_j - m).
  A6  A row without valid entries gives o = 0 and lse = -inf.

Padding entries are skipped: they contribute exactly nothing, whatever bytes the
reserved slot 0 or any unreferenced slot holds.  The second function models the
faulty reader the pages describe (padding clamped to slot 0, score masked, the
row still multiplied into the value product) and exists only so a test can
check that it reproduces the pages' failure pattern.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

ROW_BYTES = 656
LATENT = 512
TILE = 128
SCALE_OFF = 512
ROPE_OFF = 528


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def dequant_rows(cache: np.ndarray, slots: np.ndarray, rope_dim: int) -> np.ndarray:
    """A2: float64 K rows [n][512 + rope_dim] of the given slots."""
    rows = cache[np.asarray(slots, dtype=np.int64)]
    n = rows.shape[0]
    codes = rows[:, :LATENT]
    scales = np.ascontiguousarray(rows[:, SCALE_OFF:ROPE_OFF]).view("<f4").astype(np.float64)
    k = e4m3.decode(codes).reshape(n, 4, TILE) * scales[:, :, None]   # exact in f64
    k = k.reshape(n, LATENT)
    if rope_dim:
        rope = np.ascontiguousarray(rows[:, ROPE_OFF:ROPE_OFF + 2 * rope_dim]).view("<u2")
        k = np.concatenate([k, _bf16_to_f64(rope)], axis=1)
    return k


def valid_entries(idx_row: np.ndarray, width: int, num_slots: int) -> np.ndarray:
    """A1: the valid entries of one index row, in buffer order."""
    r = np.asarray(idx_row[:width], dtype=np.int64)
    return r[(r >= 0) & (r < num_slots)]


def sparse_mla_attn(q_bits: np.ndarray, cache: np.ndarray, idx: np.ndarray, width: int,
                    rope_dim: int, sm_scale: float, rows=None):
    """Exact sparse attention.  q_bits: bf16 bits [T][H][512 + rope_dim];
    cache: uint8 [num_slots][656]; idx: int32 [T][>= width].
    Returns (out float64 [T][H][512], lse float64 [T][H]); `rows` restricts the
    computation to the listed query rows (others are left NaN)."""
    return _attend(q_bits, cache.shape[0], lambda v: dequant_rows(cache, v, rope_dim), idx, width,
                   rope_dim, sm_scale, rows)


def sparse_mla_attn_bf16(q_bits: np.ndarray, cache_bits: np.ndarray, idx: np.ndarray, width: int,
                         rope_dim: int, sm_scale: float, rows=None):
    """The same attention over a BF16 KV cache (sglang PR 47013, Speed Tests):
    cache_bits uint16 [num_slots][512 + rope_dim] holds the K rows themselves,
    K[j][e] = bf16 value e of row j (A2 without dequantisation)."""
    assert cache_bits.shape[1] == LATENT + rope_dim
    return _attend(q_bits, cache_bits.shape[0],
                   lambda v: _bf16_to_f64(cache_bits[np.asarray(v, dtype=np.int64)]), idx, width,
                   rope_dim, sm_scale, rows)


def _attend(q_bits, num_slots, k_rows, idx, width, rope_dim, sm_scale, rows):
    """A1, A3-A6 over K rows given by k_rows(valid slots) -> float64 [n][512 + rope_dim]."""
    q = _bf16_to_f64(q_bits)
    T, H, D = q.shape
    assert D == LATENT + rope_dim
    out = np.full((T, H, LATENT), np.nan)
    lse = np.full((T, H), np.nan)
    for t in (range(T) if rows is None else rows):
        v = valid_entries(idx[t], width, num_slots)
        if v.size == 0:                                                  # A6
            out[t] = 0.0
            lse[t] = -np.inf
            continue
        k = k_rows(v)                                                    # A2
        s = float(sm_scale) * (q[t] @ k.T)                               # A3  [H][n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        out[t] = (e / z) @ k[:, :LATENT]                                 # A4, A5
        lse[t] = m[:, 0] + np.log(z[:, 0])
    return out, lse


def clamped_gather_attn(q_bits: np.ndarray, cache: np.ndarray, idx: np.ndarray, width: int,
                        rope_dim: int, sm_scale: float):
    """The faulty reader of sglang PR 39288, Root cause (1): every padding
    index is clamped to slot 0 and gathered, its score is masked to -1e30, and
    the gathered row still enters the value product with weight 0, so
    0 * NaN = NaN whenever slot 0 holds NaN codes.  Negative control only."""
    q = _bf16_to_f64(q_bits)
    T, H, _ = q.shape
    out = np.zeros((T, H, LATENT))
    with np.errstate(invalid="ignore", over="ignore"):
        for t in range(T):
            r = np.asarray(idx[t, :width], dtype=np.int64)
            pad = r < 0
            g = np.where(pad, 0, r)
            k = dequant_rows(cache, g, rope_dim)
            s = float(sm_scale) * (q[t] @ np.nan_to_num(k, nan=0.0, posinf=0.0, neginf=0.0).T)
            s[:, pad] = -1e30
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p = p / p.sum(axis=1, keepdims=True)
            out[t] = p @ k[:, :LATENT]
    return out
