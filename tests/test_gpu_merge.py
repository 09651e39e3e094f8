"""HIP log-sum-exp merge vs the float64 oracle: on the same bf16 partial
results (ragged sizes, empty parts holding NaN, every part empty), and end to
end as context-parallel decoding would use it: each owner of a share of the
cache slots attends over its own top-k entries, then the merge recombines, to
the attention parity bar against the oracle over the whole row."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from oracle import merge as oracle_merge
from tests.gpu_util import DEV, assert_parity, bf16_dev, build_cache, oracle_for, to_f64

pytestmark = pytest.mark.gpu


def _parts(seed, P, T, H, empty_frac=0.2):
    rng = np.random.default_rng(seed)
    o = wl.normal_bf16(rng, (P, T, H, 512))
    l = rng.uniform(-8.0, 8.0, size=(P, T, H)).astype(np.float32)
    empty = rng.random((P, T, H)) < empty_frac
    l[empty] = -np.inf
    o[empty] = 0x7FC0                    # an empty part's output is never read
    if T > 1:
        l[:, 1, 0] = -np.inf             # a (row, head) with every part empty
    return o, l


@pytest.mark.parametrize("P,T,H", [(1, 3, 16), (2, 5, 16), (8, 7, 16), (13, 2, 5), (4, 33, 128)])
def test_merge_matches_oracle(P, T, H):
    print(f"merge P={P} T={T} H={H}", flush=True)
    o_bits, l = _parts(100 + P, P, T, H)
    out, lse = smla.merge(bf16_dev(o_bits), torch.from_numpy(l).to(DEV))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_merge.merge(oracle_merge.bf16_to_f64(o_bits), l.astype(np.float64))
    g = to_f64(out)
    assert np.all(np.isfinite(g))
    # fp32 weights and sums (~1e-6 relative), then one bf16 rounding (2^-9)
    live = np.isfinite(l)[..., None] & np.ones((1, 1, 1, 512), dtype=bool)
    omax = np.abs(oracle_merge.bf16_to_f64(o_bits))[live].max()   # empty parts hold NaN
    bound = 2.0**-8 * np.abs(ref_out) + 1e-5 * omax
    assert np.all(np.abs(g - ref_out) <= bound)
    gl = lse.cpu().numpy().astype(np.float64)
    inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(gl), inf)
    assert np.abs(gl[~inf] - ref_lse[~inf]).max() <= 1e-5 * max(1.0, np.abs(ref_lse[~inf]).max())
    assert np.all(g[inf] == 0.0)
    if P == 1:   # one part: its bf16 output comes back bit for bit where it is not empty
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[~inf], o_bits[0][~inf])


@pytest.mark.parametrize("P,rope", [(4, False), (8, True)])
def test_context_parallel_decode_end_to_end(P, rope):
    """Slots are owned round-robin by P ranks; rank p attends over the entries
    it owns (the rest of the row set to -1), the merge recombines."""
    print(f"dcp P={P} rope={rope}", flush=True)
    T = 24
    if rope:
        cfg = wl.config_rope_decode(T, seed=300 + P, num_slots=16384, ctx=(512, 16384))
    else:
        cfg = wl.config_nope_decode(T, seed=300 + P, num_slots=16384, ctx=(512, 16384))
    cache = build_cache(cfg)
    idx = cfg["idx"]
    q = bf16_dev(cfg["q"])
    outs, lses = [], []
    for p in range(P):
        own = np.where((idx >= 0) & (idx % P == p), idx, -1).astype(np.int32)
        o, l = smla.attn(q, cache, torch.from_numpy(own).to(DEV), cfg["sm_scale"], cfg["rope_dim"])
        outs.append(o)
        lses.append(l)
    out, lse = smla.merge(torch.stack(outs).contiguous(), torch.stack(lses).contiguous())
    torch.cuda.synchronize()
    rows = range(T)
    ref_out, ref_lse = oracle_for(cfg, rows)
    assert_parity(out, lse, ref_out, ref_lse, rows)
    # and the merge agrees with the single call over the whole row
    full, full_lse = smla.attn(q, cache, torch.from_numpy(idx).to(DEV), cfg["sm_scale"], cfg["rope_dim"])
    torch.cuda.synchronize()
    assert np.abs(to_f64(out) - to_f64(full)).max() <= 2e-2
