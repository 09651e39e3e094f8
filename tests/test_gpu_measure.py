"""smla_gather_rows_probe reads exactly the bytes an attention call gathers:
its XOR fold equals the host's XOR of the first 528 (NoPE) or 656 (RoPE)
bytes of every listed row, with out-of-range entries skipped."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_fp8_amd as smla
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rope_dim,n", [(0, 5000), (64, 5000), (0, 1), (64, 300_001)])
def test_probe_reads_the_gathered_bytes(rope_dim, n):
    rng = np.random.default_rng(900 + n + rope_dim)
    num_slots = 40_000
    host = rng.integers(0, 256, size=(num_slots, 656), dtype=np.uint8)
    slots = rng.integers(0, num_slots, size=n).astype(np.int32)
    if n > 10:
        slots[::7] = -1                          # skipped
        slots[3::11] = num_slots + 5             # skipped
    cache = torch.from_numpy(host).to(DEV)
    sink = smla.gather_rows_probe(cache, torch.from_numpy(slots).to(DEV), rope_dim)
    torch.cuda.synchronize()
    rb = 656 if rope_dim else 528
    ok = slots[(slots >= 0) & (slots < num_slots)]
    words = host[ok, :rb].copy().view("<u4")
    want = np.bitwise_xor.reduce(words.ravel()) if words.size else np.uint32(0)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == np.uint32(want)
