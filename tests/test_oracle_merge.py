"""Pins of the oracle's log-sum-exp merge against the attention definition
itself: attention over a row's entries equals the merge of attention over any
partition of them into owners (some owners empty), plus closed forms and the
empty-part rules."""
import numpy as np
import pytest

import workloads as wl
from oracle import attention as A
from oracle import merge as M
from oracle import writer


def _setup(seed, rope_dim, n_valid=150, num_slots=512, H=4, W=192):
    rng = np.random.default_rng(seed)
    lat, rope, slots = wl.cache_rows(rng, num_slots, rope_dim)
    cache = np.zeros((num_slots, 656), dtype=np.uint8)
    writer.kv_write(cache, lat, rope, slots)
    cache[0] = wl.slot0_bytes(rng, "ff")
    q = wl.normal_bf16(rng, (1, H, 512 + rope_dim))
    idx = np.full((1, W), -1, dtype=np.int32)
    pos = rng.choice(W, size=n_valid, replace=False)          # padding anywhere
    idx[0, pos] = rng.choice(np.arange(1, num_slots), size=n_valid, replace=False)
    return rng, cache, q, idx, float(1.0 / np.sqrt(512 + rope_dim))


@pytest.mark.parametrize("rope_dim,P,seed", [(64, 2, 1), (64, 5, 2), (0, 8, 3), (0, 3, 4)])
def test_merge_of_a_partition_equals_attention_over_the_union(rope_dim, P, seed):
    rng, cache, q, idx, sm = _setup(seed, rope_dim)
    full_out, full_lse = A.sparse_mla_attn(q, cache, idx, idx.shape[1], rope_dim, sm)
    owner = rng.integers(0, P, size=idx.shape[1])
    owner[owner == P - 1] = 0            # owner P-1 gets nothing: an empty part
    parts_out, parts_lse = [], []
    for p in range(P):
        part_idx = np.where(owner[None, :] == p, idx, -1).astype(np.int32)
        o, l = A.sparse_mla_attn(q, cache, part_idx, idx.shape[1], rope_dim, sm)
        parts_out.append(o)
        parts_lse.append(l)
    assert np.all(np.isneginf(parts_lse[P - 1]))
    out, lse = M.merge(np.stack(parts_out), np.stack(parts_lse))
    scale = np.abs(full_out).max()
    assert np.abs(out - full_out).max() <= 1e-12 * scale
    assert np.abs(lse - full_lse).max() <= 1e-12 * np.abs(full_lse).max()


def test_two_part_closed_form():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((1, 1, 512))
    b = rng.standard_normal((1, 1, 512))
    out, lse = M.merge(np.stack([a, b]), np.array([[[0.0]], [[np.log(3.0)]]]))
    # weights 1/4 and 3/4, lse = ln 4
    assert np.abs(out[0, 0] - (0.25 * a[0, 0] + 0.75 * b[0, 0])).max() <= 1e-15
    assert abs(lse[0, 0] - np.log(4.0)) <= 1e-15


def test_single_part_is_returned_unchanged():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((1, 3, 2, 512))
    l = rng.uniform(-20, 20, size=(1, 3, 2))
    out, lse = M.merge(a, l)
    assert np.array_equal(out, a[0]) and np.array_equal(lse, l[0])


def test_empty_parts_weigh_nothing_and_are_not_read():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((3, 2, 2, 512))
    l = rng.uniform(-3, 3, size=(3, 2, 2))
    a_nan = a.copy()
    a_nan[1] = np.nan                     # an empty owner's output holds garbage
    l_empty = l.copy()
    l_empty[1] = -np.inf
    out, lse = M.merge(a_nan, l_empty)
    ref_out, ref_lse = M.merge(a[[0, 2]], l[[0, 2]])
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)
    # every part empty: zeros and -inf
    out, lse = M.merge(a_nan, np.full_like(l, -np.inf))
    assert np.array_equal(out, np.zeros_like(out)) and np.all(np.isneginf(lse))


def test_order_of_parts_does_not_matter():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((6, 2, 3, 512))
    l = rng.uniform(-30, 30, size=(6, 2, 3))
    out, lse = M.merge(a, l)
    perm = rng.permutation(6)
    out2, lse2 = M.merge(a[perm], l[perm])
    assert np.abs(out - out2).max() <= 1e-13 and np.abs(lse - lse2).max() <= 1e-13
