"""HIP page re-split vs the oracle, byte for byte: fp8_ds_mla rows (656 B) and
BF16 rows (1,024 B), padded destination pages, touched lists with page 0 or
without it, duplicates and ignored entries; then attention over the scratch
equals attention over the pool (slots keep their numbers)."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from oracle import pages as oracle_pages
from tests.gpu_util import DEV, bf16_dev, build_cache

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("row_bytes,pad,with_page0", [(656, 0, False), (656, 48, True), (1024, 16, False), (585, 0, True)])
def test_split_byte_exact(row_bytes, pad, with_page0):
    print(f"split rb={row_bytes} pad={pad} page0={with_page0}", flush=True)
    rng = np.random.default_rng(row_bytes + pad)
    n_src = 37
    pool = rng.integers(0, 256, size=(n_src, 256 * row_bytes), dtype=np.uint8)
    pool[0] = 0xFF                                       # NaN bytes in source page 0
    touched = rng.choice(np.arange(1, n_src), size=12, replace=False).astype(np.int32)
    touched = np.concatenate([touched, touched[:2], np.array([-1, n_src, 10_000], dtype=np.int32)])
    if with_page0:
        touched = np.concatenate([touched, np.array([0], dtype=np.int32)])
    dst_h = np.zeros((4 * n_src, 64 * row_bytes + pad), dtype=np.uint8)   # zero-filled at allocation
    dst = torch.from_numpy(dst_h).to(DEV)
    smla.split_pages_64(torch.from_numpy(pool).to(DEV), torch.from_numpy(touched).to(DEV), dst, row_bytes)
    torch.cuda.synchronize()
    oracle_pages.split_pages_64(pool, touched, dst_h, row_bytes)
    assert np.array_equal(dst.cpu().numpy(), dst_h)
    assert bool((dst[0, :64 * row_bytes] == 0xFF).all()) == with_page0   # slot 0 finite unless page 0 copied


def test_attention_over_the_scratch_matches_the_pool():
    cfg = wl.config_nope_decode(8, seed=500, num_slots=256 * 64, ctx=(256, 8192))
    cache = build_cache(cfg, check_slots=np.arange(1, 64))
    n_src = cfg["num_slots"] // 256
    idx = cfg["idx"]
    used = np.unique(idx[idx >= 0]) // 256
    scratch = torch.zeros((4 * n_src, 64 * 656), dtype=torch.uint8, device=DEV)
    smla.split_pages_64(cache.view(n_src, 256 * 656), torch.from_numpy(used.astype(np.int32)).to(DEV), scratch)
    q = bf16_dev(cfg["q"])
    ti = torch.from_numpy(idx).to(DEV)
    a, la = smla.attn(q, cache, ti, cfg["sm_scale"], 0)
    b, lb = smla.attn(q, scratch.view(-1, 656), ti, cfg["sm_scale"], 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
