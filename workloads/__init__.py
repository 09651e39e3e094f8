"""Seeded synthetic inputs for the sparse-MLA writer and attention.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no quantisation, no attention), so that the CPU oracle and
the HIP path can both be fed from it without sharing any of the computation.

Shapes follow the workloads the source pages describe:

* sglang PR 47013 (zero-RoPE writer skips slot 0), Speed Tests: writer calls of
  1,024 and 8,192 bf16 rows of 512 values, with one row in four a padding row
  for slot 0; decode at 16 heads, d_v 512, top-k 2048, 1-256 tokens.
* sglang PR 39288 (SM120 page-split scratch), Root cause and kernel-harness
  table: 64-token pages, H=16, -1 padding, slot 0 holding 0xFF, random or zero
  bytes, prefill T=65 / decode T=64 boundary.
* vLLM PR 55277 (NoPE sparse MLA on SM120), Purpose (1) and (2): the 656-byte
  fp8_ds_mla row also for NoPE models, and a top-k buffer of width 2176
  (index_topk 2048 plus a 128-wide tail).

All arrays are numpy; bf16 values are carried as their uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

PAGE = 64               # tokens per page (sglang PR 39288, Root cause (2))
LATENT = 512            # latent width (vLLM PR 55277, Purpose (1))
ROPE = 64               # RoPE width when present
ROW_BYTES = 656         # packed fp8_ds_mla row

BF16_QNAN = np.uint16(0x7FC0)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return bits.

    Inputs are finite (the generators only draw normals)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: |u| stays below 0x7F800000 per sign, so the sum cannot wrap
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 bits of N(0,1) samples drawn in float32."""
    return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))


# --------------------------------------------------------------------------
# top-k index builders
# --------------------------------------------------------------------------

def decode_topk(rng: np.random.Generator, T: int, width: int, num_slots: int,
                ctx_lo: int, ctx_hi: int, index_topk: int = 2048) -> np.ndarray:
    """Per-token top-k slot lists for decode.

    Each token owns a context of L ~ U{ctx_lo..ctx_hi} tokens laid out on
    ceil(L/64) distinct random pages (page 0 is reserved, as sglang reserves
    full-pool page 0).  min(L, index_topk) distinct positions of the context are
    drawn without replacement in random order and mapped to their slots; the
    rest of the row, up to `width`, is -1.
    """
    n_pages = num_slots // PAGE
    out = np.full((T, width), -1, dtype=np.int32)
    for t in range(T):
        L = int(rng.integers(ctx_lo, ctx_hi + 1))
        pages = rng.choice(n_pages - 1, size=(L + PAGE - 1) // PAGE, replace=False) + 1
        n = min(L, index_topk, width)
        pos = rng.choice(L, size=n, replace=False)
        out[t, :n] = (pages[pos // PAGE] * PAGE + pos % PAGE).astype(np.int32)
    return out


def prefill_topk(rng: np.random.Generator, T: int, width: int, num_slots: int):
    """Top-k lists of one causal sequence of T tokens.

    The sequence sits on ceil(T/64) distinct random pages (page 0 excluded).
    Row t lists the slots of tokens 0..t (all of them while t < width, else a
    random subset of `width`), shuffled, then -1.  Returns (idx, seq_slots)."""
    n_pages = num_slots // PAGE
    pages = rng.choice(n_pages - 1, size=(T + PAGE - 1) // PAGE, replace=False) + 1
    seq_slots = (pages[np.arange(T) // PAGE] * PAGE + np.arange(T) % PAGE).astype(np.int32)
    out = np.full((T, width), -1, dtype=np.int32)
    for t in range(T):
        n = min(t + 1, width)
        sel = rng.choice(t + 1, size=n, replace=False)
        out[t, :n] = seq_slots[sel]
    return out, seq_slots


def disjoint_topk(rng: np.random.Generator, T: int, width: int, num_slots: int) -> np.ndarray:
    """T rows of `width` slots, pairwise disjoint across the whole batch (slot 0 excluded)."""
    assert T * width <= num_slots - 1
    perm = rng.permutation(num_slots - 1)[: T * width] + 1
    return perm.reshape(T, width).astype(np.int32)


# --------------------------------------------------------------------------
# whole workloads
# --------------------------------------------------------------------------

def cache_rows(rng: np.random.Generator, num_slots: int, rope_dim: int):
    """bf16 latent and RoPE rows for every slot 1..num_slots-1 (row i -> slot i+1)."""
    n = num_slots - 1
    latent = normal_bf16(rng, (n, LATENT))
    rope = normal_bf16(rng, (n, rope_dim)) if rope_dim else None
    slots = np.arange(1, num_slots, dtype=np.int64)
    return latent, rope, slots


def slot0_bytes(rng: np.random.Generator, poison: str) -> np.ndarray:
    """656 bytes for the reserved slot: 'ff', '7f', 'zero' or 'random'."""
    if poison == "ff":
        return np.full(ROW_BYTES, 0xFF, dtype=np.uint8)
    if poison == "7f":
        return np.full(ROW_BYTES, 0x7F, dtype=np.uint8)
    if poison == "zero":
        return np.zeros(ROW_BYTES, dtype=np.uint8)
    if poison == "random":
        return rng.integers(0, 256, size=ROW_BYTES, dtype=np.uint8)
    raise ValueError(poison)


def config_tiny(seed: int = 1) -> dict:
    """Tiny decode: 4 pages x 64 = 256 slots, rope 64, slot 0 = 0xFF, T=2, H=4,
    top-k 128 with 77 distinct random slots in 1..255 then 51 x -1."""
    rng = np.random.default_rng(seed)
    num_slots, rope_dim, T, H, W = 256, ROPE, 2, 4, 128
    latent, rope, slots = cache_rows(rng, num_slots, rope_dim)
    q = normal_bf16(rng, (T, H, LATENT + rope_dim))
    n_pad = int(np.floor(0.4 * W))
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        idx[t, : W - n_pad] = rng.choice(np.arange(1, num_slots), size=W - n_pad, replace=False)
    return dict(num_slots=num_slots, rope_dim=rope_dim, T=T, H=H, W=W,
                latent=latent, rope=rope, slots=slots, q=q, idx=idx,
                sm_scale=float(1.0 / np.sqrt(LATENT + rope_dim)),
                slot0=slot0_bytes(rng, "ff"))


def config_nope_decode(T: int, seed: int | None = None, num_slots: int = 131072,
                       H: int = 16, ctx=(1024, 65536), W: int = 2176) -> dict:
    """GLM-style NoPE decode: rope 0, H=16, 131,072-slot cache, contexts
    U{1k..64k}, width 2176 (2048 + a 128-wide tail of -1), slot 0 = 0x7F."""
    rng = np.random.default_rng(20 + T if seed is None else seed)
    latent, rope, slots = cache_rows(rng, num_slots, 0)
    q = normal_bf16(rng, (T, H, LATENT))
    idx = decode_topk(rng, T, W, num_slots, ctx[0], ctx[1])
    return dict(num_slots=num_slots, rope_dim=0, T=T, H=H, W=W,
                latent=latent, rope=rope, slots=slots, q=q, idx=idx,
                sm_scale=float(1.0 / np.sqrt(LATENT)), slot0=slot0_bytes(rng, "7f"))


def config_rope_decode(T: int, seed: int | None = None, num_slots: int = 262144,
                       H: int = 16, ctx=(2048, 131072), W: int = 2048) -> dict:
    """DeepSeek-style RoPE decode: rope 64, H=16, top-k 2048, contexts
    U{2k..128k}, 262,144-slot cache, slot 0 random bytes."""
    rng = np.random.default_rng(30 + T if seed is None else seed)
    latent, rope, slots = cache_rows(rng, num_slots, ROPE)
    q = normal_bf16(rng, (T, H, LATENT + ROPE))
    idx = decode_topk(rng, T, W, num_slots, ctx[0], ctx[1])
    return dict(num_slots=num_slots, rope_dim=ROPE, T=T, H=H, W=W,
                latent=latent, rope=rope, slots=slots, q=q, idx=idx,
                sm_scale=float(1.0 / np.sqrt(LATENT + ROPE)), slot0=slot0_bytes(rng, "random"))


def config_prefill(T: int, seed: int | None = None, num_slots: int = 131072,
                   H: int = 16, W: int = 2048) -> dict:
    """Sparse prefill: T query rows of one causal sequence; row t lists the
    slots of tokens <= t then -1; rope 64; slot 0 random bytes."""
    rng = np.random.default_rng(40 + T if seed is None else seed)
    latent, rope, slots = cache_rows(rng, num_slots, ROPE)
    q = normal_bf16(rng, (T, H, LATENT + ROPE))
    idx, seq = prefill_topk(rng, T, W, num_slots)
    return dict(num_slots=num_slots, rope_dim=ROPE, T=T, H=H, W=W,
                latent=latent, rope=rope, slots=slots, q=q, idx=idx, seq_slots=seq,
                sm_scale=float(1.0 / np.sqrt(LATENT + ROPE)), slot0=slot0_bytes(rng, "random"))


def config_disjoint(T: int = 64, seed: int = 60, num_slots: int = 262144,
                    H: int = 16, W: int = 2048, rope_dim: int = ROPE, listed_only: bool = False,
                    n_valid: int | None = None) -> dict:
    """Decode whose top-k sets are pairwise disjoint across the batch, so
    gathered bytes equal unique bytes (a control against cache reuse).

    Default: the RoPE decode shape at T=64 on a 262,144-slot cache whose every
    row is written.  With listed_only=True only the slots the top-k lists name
    get rows (`slots` then holds those slot ids in ascending order, row i of
    `latent` / `rope` going to slots[i]), which keeps a cache of a million
    slots cheap to build; n_valid < W leaves the last W - n_valid entries of
    every row -1 (the 2176-wide NoPE buffer with its 128-wide tail)."""
    rng = np.random.default_rng(seed)
    nv = W if n_valid is None else n_valid
    if listed_only:
        body = disjoint_topk(rng, T, nv, num_slots)
        slots = np.sort(body.ravel()).astype(np.int64)
        latent = normal_bf16(rng, (slots.size, LATENT))
        rope = normal_bf16(rng, (slots.size, rope_dim)) if rope_dim else None
        q = normal_bf16(rng, (T, H, LATENT + rope_dim))
    else:
        latent, rope, slots = cache_rows(rng, num_slots, rope_dim)
        q = normal_bf16(rng, (T, H, LATENT + rope_dim))
        body = disjoint_topk(rng, T, nv, num_slots)
    idx = np.full((T, W), -1, dtype=np.int32)
    idx[:, :nv] = body
    return dict(num_slots=num_slots, rope_dim=rope_dim, T=T, H=H, W=W,
                latent=latent, rope=rope, slots=slots, q=q, idx=idx,
                sm_scale=float(1.0 / np.sqrt(LATENT + rope_dim)),
                slot0=slot0_bytes(rng, "random" if rope_dim else "7f"))


def config_disjoint_t256(rope_dim: int) -> dict:
    """The headline decode batch (256 tokens, H=16, top-k 2048) with pairwise
    disjoint top-k sets on a 1,048,576-slot cache: 524,288 distinct slots, so
    every gathered row is read once per call.  NoPE rows use the 2176-wide
    buffer (2048 entries, then a 128-wide -1 tail), RoPE rows a 2048-wide one."""
    if rope_dim:
        return config_disjoint(T=256, seed=61, num_slots=1 << 20, W=2048, rope_dim=ROPE,
                               listed_only=True)
    return config_disjoint(T=256, seed=62, num_slots=1 << 20, W=2176, rope_dim=0,
                           listed_only=True, n_valid=2048)


def config_writer(N: int = 8192, rope_dim: int = ROPE, seed: int = 50,
                  num_slots: int = 131072, pad_frac: float = 0.25,
                  shuffle: bool = False) -> dict:
    """Standalone writer call: N rows, the trailing pad_frac of which are padding
    rows for slot 0 with bf16 NaN inputs; the rest go to distinct random
    slots >= 1.  The cache starts as 0xA5 except slot 0, which is zero."""
    rng = np.random.default_rng(seed)
    n_pad = int(round(N * pad_frac))
    n_real = N - n_pad
    latent = normal_bf16(rng, (N, LATENT))
    rope = normal_bf16(rng, (N, rope_dim)) if rope_dim else None
    slots = np.zeros(N, dtype=np.int64)
    slots[:n_real] = rng.choice(num_slots - 1, size=n_real, replace=False) + 1
    latent[n_real:] = BF16_QNAN
    if rope is not None:
        rope[n_real:] = BF16_QNAN
    if shuffle:
        perm = rng.permutation(N)
        latent, slots = latent[perm], slots[perm]
        if rope is not None:
            rope = rope[perm]
    cache = np.full((num_slots, ROW_BYTES), 0xA5, dtype=np.uint8)
    cache[0] = 0
    return dict(num_slots=num_slots, rope_dim=rope_dim, N=N, latent=latent,
                rope=rope, slots=slots, cache=cache)


def config_random_shape(seed: int) -> dict:
    """A call of random shape for sweep tests: rope 0 or 64, T, H and the
    buffer width W drawn across the launch plan's boundaries (one or many
    splits, two or three merged in the launch, four-wavefront workgroups,
    buffers wider than one scan), a small cache, and top-k rows whose valid
    count, padding positions, duplicates and out-of-range entries vary per row.
    `idx` may be wider than W (its extra columns are junk the call must not
    read); `stride_extra` says by how much.  Slot 0 is listed only when its
    bytes are zeros."""
    rng = np.random.default_rng(900_000 + seed)
    rope_dim = int(rng.choice([0, ROPE]))
    T = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 65, 100, 128, 129, 200, 256, 257, 300, 513]))
    H = int(rng.choice([1, 3, 8, 16, 17, 32, 48]))
    W = int(rng.choice([1, 7, 64, 65, 300, 2048, 2176, 2304, 2305, 3000]))
    num_slots = int(rng.choice([1024, 2048, 4096]))
    stride_extra = int(rng.choice([0, 0, 5]))
    poison = str(rng.choice(["ff", "7f", "random", "zero"]))
    # slot 0 is listed only when it holds zeros: it is read like any other
    # slot, and NaN-coded bytes there would make the listing rows NaN
    lo = 0 if poison == "zero" else 1
    latent, rope, slots = cache_rows(rng, num_slots, rope_dim)
    q = normal_bf16(rng, (T, H, LATENT + rope_dim))
    idx = np.full((T, W + stride_extra), -1, dtype=np.int32)
    if stride_extra:
        idx[:, W:] = rng.integers(0, num_slots, size=(T, stride_extra), dtype=np.int32)
    for t in range(T):
        kind = rng.integers(0, 8)
        if kind == 0:
            n = 0                                  # an empty row
        elif kind == 1:
            n = W                                  # a full row
        else:
            n = int(rng.integers(0, W + 1))
        pos = rng.choice(W, size=n, replace=False)
        vals = rng.integers(lo, num_slots, size=n, dtype=np.int64)   # repeats included
        if n and rng.integers(0, 4) == 0:          # some out-of-range padding
            bad = rng.random(n) < 0.1
            vals[bad] = rng.choice([-7, num_slots, num_slots + 1000, 2**31 - 1], size=int(bad.sum()))
        idx[t, pos] = vals.astype(np.int32)
    return dict(num_slots=num_slots, rope_dim=rope_dim, T=T, H=H, W=W, stride_extra=stride_extra,
                latent=latent, rope=rope, slots=slots, q=q, idx=idx,
                sm_scale=float(1.0 / np.sqrt(LATENT + rope_dim)), slot0=slot0_bytes(rng, poison))


def config_random_shape_many_heads(seed: int) -> dict:
    """config_random_shape with 64 to 128 heads (several head groups per row)
    and T up to 100: the same cache and list rules, rows of the drawn lists
    reused in turn when T exceeds their count."""
    cfg = config_random_shape(seed)
    rng = np.random.default_rng(700_000 + seed)
    H = int(rng.choice([64, 100, 127, 128]))
    T = int(rng.choice([1, 2, 3, 11, 16, 21, 32, 33, 40, 64, 65, 100]))
    cfg["q"] = normal_bf16(rng, (T, H, LATENT + cfg["rope_dim"]))
    cfg["idx"] = np.ascontiguousarray(cfg["idx"][np.arange(T) % cfg["T"]])
    cfg["T"], cfg["H"] = T, H
    return cfg
