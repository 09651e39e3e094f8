"""Pins of the oracle writer: hand-computed rows, the fp8_ds_mla byte map, the
slot-0 drop, and a library re-derivation of the quantiser."""
import os

import numpy as np
import torch

import workloads as wl
from oracle import writer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_ds_mla_row.txt")


def _layout():
    d = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            name, off, n = line.split()
            d[name] = (int(off), int(n))
    return d


def _bits(vals):
    return wl.bf16_bits_from_f32(np.asarray(vals, dtype=np.float32))


def _hand_row():
    """Tile 0: amax 448 -> scale 1; tile 1: all zero; tile 2: amax 896 -> scale 2;
    tile 3: amax 7 -> scale 1/64 (exact), with a subnormal-range element."""
    x = np.zeros(512, dtype=np.float32)
    x[0:6] = [448.0, 1.0, -1.0, 0.5, 2.0 ** -9, -(2.0 ** -11)]
    x[256:259] = [896.0, 3.0, -896.0]
    x[384:388] = [7.0, 0.25, -3.5, 2.0 ** -13]
    return x


def test_hand_computed_row():
    x = _hand_row()
    rope = np.arange(64, dtype=np.float32) - 32.0
    row = writer.encode_rows(_bits(x)[None], _bits(rope)[None])[0]
    lay = _layout()
    o, n = lay["latent_codes"]
    codes = row[o:o + n]
    assert codes[0:6].tolist() == [0x7E, 0x38, 0xB8, 0x30, 0x01, 0x80]
    assert not codes[6:128].any()
    assert not codes[128:256].any()                       # zero tile
    assert codes[256:259].tolist() == [0x7E, 0x3C, 0xFE]  # 896/2=448, 3/2=1.5
    # tile 3: scale = 7/448 = 2^-6; 7/2^-6 = 448, 0.25*64 = 16, -3.5*64 = -224,
    # 2^-13 * 64 = 2^-7 (subnormal code 4)
    assert codes[384:388].tolist() == [0x7E, 0x58, 0xF6, 0x04]
    o, n = lay["tile_scales"]
    assert row[o:o + n].view("<f4").tolist() == [1.0, 0.0, 2.0, 2.0 ** -6]
    assert bytes(row[o:o + 4]) == b"\x00\x00\x80\x3f"
    o, n = lay["rope_or_zero"]
    assert row[o:o + n].view("<u2").tolist() == _bits(rope).tolist()
    assert o + n == lay["row_bytes"][1] == row.size


def test_nope_tail_is_zero():
    rng = np.random.default_rng(3)
    lat = wl.normal_bf16(rng, (9, 512))
    rows = writer.encode_rows(lat, None)
    o, n = _layout()["rope_or_zero"]
    assert rows.shape == (9, 656) and not rows[:, o:o + n].any()
    # latent part identical to the RoPE variant's
    rows64 = writer.encode_rows(lat, wl.normal_bf16(rng, (9, 64)))
    assert np.array_equal(rows[:, :o], rows64[:, :o])


def test_library_rederivation_of_quantiser():
    """torch float32 ops (IEEE division) + torch's float8_e4m3fn cast give the
    same codes and scale bytes on N(0,1) rows."""
    rng = np.random.default_rng(4)
    lat = wl.normal_bf16(rng, (300, 512))
    rows = writer.encode_rows(lat, None)
    x = torch.from_numpy(wl.f32_from_bf16_bits(lat).copy()).view(300, 4, 128)
    scale = x.abs().amax(dim=2) / 448.0
    codes = (x / scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(rows[:, :512], codes.reshape(300, 512).numpy())
    assert np.array_equal(rows[:, 512:528].view("<f4"), scale.numpy())


def test_dequant_error_bound_and_tile_max():
    """|x - E4M3(code)*scale| stays within the rounding bound of the format,
    and each tile's largest magnitude lands on +-448."""
    rng = np.random.default_rng(5)
    lat = wl.normal_bf16(rng, (200, 512))
    rows = writer.encode_rows(lat, None)
    x = wl.f32_from_bf16_bits(lat).astype(np.float64).reshape(200, 4, 128)
    codes = torch.from_numpy(rows[:, :512].copy()).view(torch.float8_e4m3fn)
    val = codes.to(torch.float64).numpy().reshape(200, 4, 128)
    s = rows[:, 512:528].copy().view("<f4").astype(np.float64)
    k = val * s[:, :, None]
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s[:, :, None]) * (1 + 2.0 ** -20)
    assert np.all(np.abs(x - k) <= bound)
    imax = np.argmax(np.abs(x), axis=2)
    top = np.take_along_axis(np.abs(val), imax[:, :, None], axis=2)
    assert np.all(top == 448.0)


def test_slot_drop_and_untouched_bytes():
    rng = np.random.default_rng(6)
    num_slots = 64
    cache = np.full((num_slots, 656), 0xA5, dtype=np.uint8)
    cache[0] = 0
    lat = wl.normal_bf16(rng, (6, 512))
    rope = wl.normal_bf16(rng, (6, 64))
    slots = np.array([0, 7, -1, num_slots, 0, 63], dtype=np.int64)
    lat[[0, 2, 3, 4]] = wl.BF16_QNAN           # dropped rows hold NaN
    rope[[0, 2, 3, 4]] = wl.BF16_QNAN
    keep = writer.kv_write(cache, lat, rope, slots)
    assert keep.tolist() == [False, True, False, False, False, True]
    assert not cache[0].any()                   # reserved slot stays zero
    want = writer.encode_rows(lat[[1, 5]], rope[[1, 5]])
    assert np.array_equal(cache[7], want[0]) and np.array_equal(cache[63], want[1])
    others = np.setdiff1d(np.arange(1, num_slots), [7, 63])
    assert np.all(cache[others] == 0xA5)


def test_writer_workload_shape():
    cfg = wl.config_writer(N=1024, rope_dim=0, num_slots=4096)
    cache = cfg["cache"].copy()
    keep = writer.kv_write(cache, cfg["latent"], cfg["rope"], cfg["slots"])
    assert keep.sum() == 768
    assert not cache[0].any()
    written = cfg["slots"][keep]
    assert not cache[written, 528:].any()
    untouched = np.setdiff1d(np.arange(1, 4096), written)
    assert np.all(cache[untouched] == 0xA5)


def _slot_checks(cache, cfg):
    """The checks of the writer workload: slot 0 left zero, the NoPE tail of
    every written row zero, every other slot still 0xA5."""
    written = cfg["slots"][cfg["slots"] > 0]
    ok_slot0 = not cache[0].any()
    ok_tail = cfg["rope_dim"] == 64 or not cache[written, 528:].any()
    others = np.ones(cfg["num_slots"], dtype=bool)
    others[0] = False
    others[written] = False
    ok_rest = bool((cache[others] == 0xA5).all())
    return ok_slot0, ok_tail, ok_rest


def test_negative_control_writer_without_the_slot0_skip():
    """sglang PR 47013 (Modifications; Speed Tests, writer table with a quarter
    of the rows aimed at slot 0): the check "slot 0 left zero" fails for the
    writer before the fix and passes for the writer that drops slot-0 rows.
    The pre-fix writer fills slot 0 with NaN codes (the padding rows carry NaN),
    which the clamp-to-slot-0 reader then turns into NaN output in exactly the
    rows that hold a -1 (sglang PR 39288, Root cause (1))."""
    from oracle import attention
    for rope_dim in (0, 64):
        cfg = wl.config_writer(N=8192, rope_dim=rope_dim)
        good = cfg["cache"].copy()
        writer.kv_write(good, cfg["latent"], cfg["rope"], cfg["slots"])
        assert _slot_checks(good, cfg) == (True, True, True)
        bad = cfg["cache"].copy()
        writer.unfiltered_kv_write(bad, cfg["latent"], cfg["rope"], cfg["slots"])
        ok_slot0, ok_tail, ok_rest = _slot_checks(bad, cfg)
        assert not ok_slot0 and ok_tail and ok_rest
        # the NaN padding row became NaN codes and NaN scales in slot 0
        assert set(np.unique(bad[0, :512] & 0x7F).tolist()) == {0x7F}
        assert np.isnan(bad[0, 512:528].view("<f4")).all()
        # rows 1.. of the real slots are identical under both writers
        assert np.array_equal(bad[1:], good[1:])
    # the faulty reader over the pre-fix cache: NaN rows are exactly the rows with a -1
    rng = np.random.default_rng(3)
    written = cfg["slots"][cfg["slots"] > 0]
    T, H, W = 6, 4, 64
    idx = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = W if t % 2 == 0 else W - 5 * t
        idx[t, :n] = rng.choice(written, size=n, replace=False)
    q = wl.normal_bf16(rng, (T, H, 576))
    o_bad = attention.clamped_gather_attn(q, bad, idx, W, 64, 1 / 24)
    o_good, _ = attention.sparse_mla_attn(q, good, idx, W, 64, 1 / 24)
    has_pad = (idx < 0).any(axis=1)
    assert np.array_equal(np.isnan(o_bad).any(axis=(1, 2)), has_pad)
    assert np.isfinite(o_good).all()


def test_writer_scale_sweep_covers_the_fast_path_threshold():
    """The exponents of the GPU writer sweep reach scales on both sides of
    2^-60 (the kernel's fast-path bound), and at each swept exponent the 128
    maxima give 128 distinct float32 scales."""
    from tests.test_gpu_writer import SWEEP_EXPONENTS
    for e in SWEEP_EXPONENTS:
        amax = [((e << 7) | m) for m in range(128) if (e, m) != (0, 0)]
        f = (np.array(amax, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
        scales = (f / 448.0).astype(np.float32)
        assert np.unique(scales).size == len(amax)
        if e == 75:
            assert (scales >= 2.0 ** -60).sum() == 32 and (scales < 2.0 ** -60).sum() == 96
