"""Calls captured in a HIP graph and replayed: a decode step (the writer's new
rows, then attention over lists that hold them) and a sparse prefill.  Every
replay, with eager calls on the same buffers and synchronisations between
replays, gives the eager call's bytes; the eager step itself meets the oracle
bar on the updated cache."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from tests.gpu_util import DEV, assert_parity, bf16_dev, build_cache, oracle_for, rows_of

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _new_slots(idx: np.ndarray) -> np.ndarray:
    """One slot per token, taken from its own list, all distinct (a write call
    with repeated slots leaves any one of the rows)."""
    taken, out = set(), []
    for row in idx:
        for s in row[row >= 1]:
            if int(s) not in taken:
                taken.add(int(s))
                out.append(int(s))
                break
        else:
            raise AssertionError("a token's list has no slot left to write")
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("T", [1, 16, 100, 256])
def test_decode_step_graph_replays(T):
    """T = 1 and 16 run the split plan and its merge kernel, T = 100 two splits
    merged inside the launch (whose arrival words each replay must leave
    clean, also with eager calls on the same workspace between replays), and
    T = 256 one split per row."""
    print(f"graph decode step T={T}", flush=True)
    cfg = wl.config_nope_decode(T, seed=900 + T, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    rng = np.random.default_rng(77 + T)
    new_slots = _new_slots(cfg["idx"])
    new_lat = wl.normal_bf16(rng, (T, wl.LATENT))
    other_lat = wl.normal_bf16(rng, (T, wl.LATENT))
    W = cfg["W"]
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(DEV)
    slots = torch.from_numpy(new_slots).to(DEV)
    lat, lat_other = bf16_dev(new_lat), bf16_dev(other_lat)
    out = torch.empty((T, cfg["H"], wl.LATENT), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, cfg["H"]), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(16, smla.workspace_size(T, cfg["H"], W, 0)), dtype=torch.uint8, device=DEV)

    def step():
        smla.kv_write(lat, None, slots, cache)
        smla.attn(q, cache, idx, cfg["sm_scale"], 0, topk_capacity=W, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()

    # the eager step against the oracle over the cache with the new rows
    upd = dict(cfg)
    upd["latent"] = cfg["latent"].copy()
    upd["latent"][rows_of(cfg, new_slots)] = new_lat
    rows = list(range(T)) if T <= 16 else list(range(0, T, 51))
    ref_o, ref_l = oracle_for(upd, rows)
    assert_parity(ref_out, ref_lse, ref_o, ref_l, rows)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(REPLAYS):
        # eager work on the same buffers: other rows into the same slots, and
        # an attention call over them into fresh outputs
        smla.kv_write(lat_other, None, slots, cache)
        o2, _ = smla.attn(q, cache, idx, cfg["sm_scale"], 0, topk_capacity=W, workspace=ws)
        out.zero_()
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        assert not torch.equal(o2, ref_out), "the eager call between replays saw the same rows"
        g.replay()
        if rep % 2:
            g.replay()          # back-to-back replays, no host sync between
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: output differs from the eager step"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse differs from the eager step"


def test_prefill_graph_replays():
    """Sparse prefill of 300 rows (four-wavefront workgroups, one split per
    row) captured alone; replays match the eager call bit for bit."""
    T = 300
    print(f"graph prefill T={T}", flush=True)
    cfg = wl.config_prefill(T, seed=950, num_slots=4096)
    cache = build_cache(cfg)
    W = cfg["idx"].shape[1]
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(DEV)
    out = torch.empty((T, cfg["H"], wl.LATENT), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((T, cfg["H"]), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(16, smla.workspace_size(T, cfg["H"], W, cfg["rope_dim"])), dtype=torch.uint8,
                     device=DEV)

    def call():
        smla.attn(q, cache, idx, cfg["sm_scale"], cfg["rope_dim"], topk_capacity=W, out=out, lse=lse,
                  workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    q_other = bf16_dev(wl.normal_bf16(np.random.default_rng(5), tuple(q.shape)))
    for rep in range(REPLAYS):
        smla.attn(q_other, cache, idx, cfg["sm_scale"], cfg["rope_dim"], topk_capacity=W)
        out.zero_()
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: output differs from the eager call"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse differs from the eager call"
