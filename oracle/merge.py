"""Merge of partial attention results by log-sum-exp, float64 reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: when the top-k entries of a query row are split over P
owners (the context-parallel decode ranks of sglang PR 47013, Motivation, or
the splits of the split-K decode kernel of sglang PR 39288, Motivation), each
owner p returns its normalised output O_p and lse_p = ln sum_{j in p} exp(s_j).
Since sum_j exp(s_j) v_j = sum_p exp(lse_p) O_p, the full result is

  lse = ln sum_p exp(lse_p),     O = sum_p exp(lse_p - lse) O_p,

with lse_p = -inf (an owner without valid entries) contributing nothing; if
every part is empty, O = 0 and lse = -inf (the empty-row rule of the
attention oracle).
"""
from __future__ import annotations

import numpy as np

LATENT = 512


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def merge(part_out: np.ndarray, part_lse: np.ndarray):
    """part_out float64 [P][T][H][512], part_lse float64 [P][T][H].
    Returns (out float64 [T][H][512], lse float64 [T][H])."""
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    P, T, H = part_lse.shape
    out = np.zeros((T, H, part_out.shape[-1]))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        for h in range(H):
            l = part_lse[:, t, h]
            live = l != -np.inf
            if not live.any():
                continue
            m = l[live].max()
            lse[t, h] = m + np.log(np.exp(l[live] - m).sum())
            w = np.exp(l[live] - lse[t, h])
            out[t, h] = w @ part_out[live, t, h]
    return out, lse
