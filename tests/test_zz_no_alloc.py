"""sparse_mla_attn_noalloc (split partials in the library's per-GPU scratch)
against sparse_mla_attn (caller workspace): identical bits, on two calls in a
row with the second one smaller, and the oracle bar; sizes beyond the scratch
are refused before any launch."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_fp8_amd as smla
import workloads as wl
from tests.gpu_util import DEV, assert_parity, bf16_dev, build_cache, oracle_for

pytestmark = pytest.mark.gpu


def _both(cfg, cache, T):
    q = bf16_dev(cfg["q"][:T])
    idx = torch.from_numpy(np.ascontiguousarray(cfg["idx"][:T])).to(DEV)
    ref_out, ref_lse = smla.attn(q, cache, idx, cfg["sm_scale"], cfg["rope_dim"])
    out = torch.full((T, cfg["H"], 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, cfg["H"]), float("nan"), dtype=torch.float32, device=DEV)
    before = torch.cuda.memory_allocated()
    smla.attn_noalloc(q, cache, idx, cfg["sm_scale"], cfg["rope_dim"], out, lse)
    assert torch.cuda.memory_allocated() == before
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


@pytest.mark.parametrize("kind,T1,T2", [("nope", 16, 4), ("rope", 64, 1), ("nope", 1, 256), ("nope", 100, 70)])
def test_noalloc_matches_workspace_entry_point(kind, T1, T2):
    print(f"noalloc {kind} T={T1} then T={T2}", flush=True)
    if kind == "nope":
        cfg = wl.config_nope_decode(256, seed=310, num_slots=16384, ctx=(512, 16384))
    else:
        cfg = wl.config_rope_decode(256, seed=311, num_slots=32768, ctx=(2048, 32000))
    cache = build_cache(cfg)
    for T in (T1, T2):
        assert smla.workspace_size(T, cfg["H"], cfg["W"], cfg["rope_dim"]) <= smla.NOALLOC_SCRATCH_BYTES
        out, lse, ref_out, ref_lse = _both(cfg, cache, T)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"T={T} differs"
        sub = dict(cfg)
        sub["q"], sub["idx"] = cfg["q"][:T], cfg["idx"][:T]
        o, l = oracle_for(sub, range(T))
        assert_parity(out, lse, o, l, range(T))


def test_noalloc_largest_plans_and_heads():
    """The largest split partials the narrow buffers ask for (one query row of
    128 heads, 8 head groups x 32 splits), then a 3-head call."""
    cfg = wl.config_rope_decode(4, seed=312, num_slots=8192, ctx=(2048, 8000), H=128, W=2048)
    cache = build_cache(cfg)
    for T, H in ((1, 128), (4, 128)):
        assert smla.workspace_size(T, H, 2048, 64) <= smla.NOALLOC_SCRATCH_BYTES
        out, lse, ref_out, ref_lse = _both(cfg, cache, T)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    cfg3 = dict(cfg)
    cfg3["q"] = np.ascontiguousarray(cfg["q"][:, :3])
    cfg3["H"] = 3
    out, lse, ref_out, ref_lse = _both(cfg3, cache, 2)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_noalloc_refuses_plans_beyond_the_scratch():
    T, W = 256, 65536
    assert smla.workspace_size(T, 16, W, 0) > smla.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, 16, 512), dtype=torch.bfloat16, device=DEV)
    cache = torch.zeros((64, 656), dtype=torch.uint8, device=DEV)
    idx = torch.full((T, W), -1, dtype=torch.int32, device=DEV)
    out = torch.full((T, 16, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(smla.SparseMLAError) as e:
        smla.attn_noalloc(q, cache, idx, 0.04, 0, out)
    assert e.value.code == smla.SMLA_EWORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())               # nothing was launched


@pytest.mark.parametrize("T", [16, 100])
def test_noalloc_in_a_graph(T):
    """The call captured in a HIP graph (T = 16: sixteen splits and the merge
    kernel; T = 100: two splits merged inside the launch, whose arrival words
    live in the scratch too): every replay, with eager calls that use the same
    scratch between replays, gives the workspace entry point's bytes."""
    print(f"noalloc graph T={T}", flush=True)
    cfg = wl.config_nope_decode(T, seed=313, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(DEV)
    ref_out, ref_lse = smla.attn(q, cache, idx, cfg["sm_scale"], 0)
    out = torch.empty((T, cfg["H"], 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, cfg["H"]), dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        smla.attn_noalloc(q, cache, idx, cfg["sm_scale"], 0, out, lse)
    q_other = bf16_dev(wl.normal_bf16(np.random.default_rng(9), tuple(q.shape)))
    o2 = torch.empty_like(out)
    for rep in range(4):
        smla.attn_noalloc(q_other, cache, idx, cfg["sm_scale"], 0, o2)   # same scratch, other partials
        out.zero_()
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {rep} differs"
