"""The seeded input generators produce the shapes and structure the workloads name."""
import numpy as np

import workloads as wl


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    b = wl.bf16_bits_from_f32(x)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]
    assert np.array_equal(wl.f32_from_bf16_bits(b)[:4], np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5], np.float32))


def test_tiny_config():
    c = wl.config_tiny()
    assert c["q"].shape == (2, 4, 576) and c["idx"].shape == (2, 128)
    for r in c["idx"]:
        v = r[r >= 0]
        assert v.size == 77 and np.all(r[77:] == -1)
        assert len(set(v.tolist())) == 77 and v.min() >= 1 and v.max() <= 255
    assert np.all(c["slot0"] == 0xFF) and c["latent"].shape == (255, 512)


def test_decode_topk_structure():
    rng = np.random.default_rng(0)
    idx = wl.decode_topk(rng, 8, 2176, 131072, 1024, 65536)
    for r in idx:
        v = r[r >= 0]
        assert 1024 <= v.size <= 2048 and np.all(r[v.size:] == -1)
        assert len(set(v.tolist())) == v.size and v.min() >= wl.PAGE
    assert np.all(idx[:, 2048:] == -1)


def test_prefill_topk_is_causal():
    rng = np.random.default_rng(1)
    idx, seq = wl.prefill_topk(rng, 130, 2048, 131072)
    for t in range(130):
        v = idx[t][idx[t] >= 0]
        assert sorted(v.tolist()) == sorted(seq[: t + 1].tolist())


def test_disjoint_and_writer_configs():
    d = wl.disjoint_topk(np.random.default_rng(2), 16, 64, 4096)
    assert len(set(d.ravel().tolist())) == d.size and d.min() >= 1
    w = wl.config_writer(N=1024, num_slots=4096)
    assert (w["slots"] == 0).sum() == 256 and np.all(w["latent"][768:] == wl.BF16_QNAN)
    assert len(set(w["slots"][:768].tolist())) == 768 and w["slots"][:768].min() >= 1


def test_random_shape_configs():
    """The sweep generator: deterministic per seed, shapes inside the drawn
    lists, idx at least W wide with junk only past W, slot 0 listed only when
    its bytes are zeros, and every valid entry below num_slots."""
    seen = set()
    for seed in range(64):
        a, b = wl.config_random_shape(seed), wl.config_random_shape(seed)
        assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["q"], b["q"])
        T, H, W = a["T"], a["H"], a["W"]
        assert a["idx"].shape == (T, W + a["stride_extra"])
        assert a["q"].shape == (T, H, wl.LATENT + a["rope_dim"])
        assert a["latent"].shape == (a["num_slots"] - 1, wl.LATENT)
        active = a["idx"][:, :W]
        valid = (active >= 0) & (active < a["num_slots"])
        if (active == 0).any():
            assert not a["slot0"].any()
        seen.add((T * ((H + 15) // 16) > 256, W > 2304, bool((~valid.any(axis=1)).any())))
    # the draws reach both workgroup shapes, wide buffers and empty rows
    assert {s[0] for s in seen} == {False, True}
    assert {s[1] for s in seen} == {False, True}
    assert True in {s[2] for s in seen}


def test_random_shape_many_heads_configs():
    """The many-heads draws: 64 to 128 heads, q and idx with T rows, the idx
    rows taken from the base draw in turn, and among the first 24 seeds every
    plan kind (four-wavefront workgroups, two or three splits merged in the
    launch, more splits with the merge kernel)."""
    kinds = set()
    for seed in range(24):
        a = wl.config_random_shape_many_heads(seed)
        base = wl.config_random_shape(seed)
        T, H, W = a["T"], a["H"], a["W"]
        assert 64 <= H <= 128
        assert a["q"].shape == (T, H, wl.LATENT + a["rope_dim"])
        assert a["idx"].shape == (T, W + a["stride_extra"])
        assert np.array_equal(a["idx"], base["idx"][np.arange(T) % base["T"]])
        units = T * ((H + 15) // 16)
        kinds.add("four-wave" if units > 256 else "one split" if units > 128 else
                  "fused" if units > 64 else "merge kernel")
    assert kinds >= {"four-wave", "fused", "merge kernel"}
