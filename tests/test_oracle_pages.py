"""Pins of the oracle's page re-split: the slot numbers it must keep (token
t of pool page p is slot 256p + t in both layouts), the zero page 0 of a fresh
scratch when page 0 is not touched, and the bytes outside the copies."""
import numpy as np

from oracle import pages as P


def test_every_copied_row_keeps_its_slot_number():
    rng = np.random.default_rng(1)
    rb, n_src = 656, 6
    pool = rng.integers(0, 256, size=(n_src, 256 * rb), dtype=np.uint8)
    dst = np.zeros((4 * n_src, 64 * rb), dtype=np.uint8)
    touched = np.array([1, 4, 5])
    P.split_pages_64(pool, touched, dst, rb)
    rows_pool = pool.reshape(n_src * 256, rb)              # slot s = 256p + t
    rows_dst = dst.reshape(4 * n_src * 64, rb)             # slot s = 64 q + o
    for p in touched:
        for t in range(256):
            s = 256 * p + t
            assert np.array_equal(rows_dst[s], rows_pool[s])
    for p in set(range(n_src)) - set(touched.tolist()):
        assert not rows_dst[256 * p:256 * (p + 1)].any()


def test_fresh_scratch_keeps_slot0_zero_unless_page0_is_copied():
    pool = np.full((3, 256 * 16), 0xFF, dtype=np.uint8)     # NaN bytes everywhere
    dst = np.zeros((12, 64 * 16), dtype=np.uint8)
    P.split_pages_64(pool, np.array([2, 1]), dst, 16)
    assert not dst[0].any()                                 # slot 0 finite
    P.split_pages_64(pool, np.array([0]), dst, 16)
    assert np.all(dst[0] == 0xFF)


def test_padding_and_untouched_bytes_unchanged_and_bad_entries_ignored():
    rng = np.random.default_rng(2)
    pool = rng.integers(0, 256, size=(4, 256 * 32), dtype=np.uint8)
    dst = np.full((16, 64 * 32 + 48), 0x5A, dtype=np.uint8)  # padded dst pages
    P.split_pages_64(pool, np.array([3, -1, 4, 99, 3]), dst, 32)
    assert np.all(dst[:, 64 * 32:] == 0x5A)
    assert np.all(dst[:12] == 0x5A)
    assert np.array_equal(dst[12:16, :64 * 32].reshape(-1), pool[3])
