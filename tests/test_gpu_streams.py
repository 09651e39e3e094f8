"""Calls issued on two streams at once give the bits of the same calls issued
one at a time.  Each stream has its own workspace, outputs and (for the writer)
cache; the calls share nothing else, so one stream's split partials, merge
arrival words and cache rows never meet the other's."""
import numpy as np
import pytest
import torch

import workloads as wl
import sparse_mla_attention_fp8_amd as smla
from tests.gpu_util import DEV, bf16_dev, build_cache

pytestmark = pytest.mark.gpu

# one plan of each kind: a single (row, head group) on four-wavefront
# workgroups, 16 splits and the merge kernel, 3 and 2 splits merged in the
# launch, one split per row, and more rows than one round of workgroups
SIZES = (1, 16, 70, 100, 256, 300)
REPS = 3


def test_attention_on_two_streams():
    print("attention on two streams", flush=True)
    cfg = wl.config_nope_decode(300, seed=870, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(DEV)
    W = cfg["W"]
    qs = {T: q[:T].contiguous() for T in SIZES}
    ref = {T: smla.attn(qs[T], cache, idx[:T], cfg["sm_scale"], 0) for T in SIZES}
    torch.cuda.synchronize()

    orders = (SIZES, SIZES[::-1])
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    need = max(smla.workspace_size(T, 16, W, 0) for T in SIZES)
    bufs = []
    for _ in streams:
        ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
        outs = {(r, T): torch.empty((T, 16, 512), dtype=torch.bfloat16, device=DEV)
                for r in range(REPS) for T in SIZES}
        lses = {(r, T): torch.empty((T, 16), dtype=torch.float32, device=DEV)
                for r in range(REPS) for T in SIZES}
        bufs.append((ws, outs, lses))
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    # the two streams' launches interleave call by call
    for r in range(REPS):
        for i in range(len(SIZES)):
            for s, order, (ws, outs, lses) in zip(streams, orders, bufs):
                T = order[i]
                with torch.cuda.stream(s):
                    smla.attn(qs[T], cache, idx[:T], cfg["sm_scale"], 0, out=outs[(r, T)], lse=lses[(r, T)],
                              workspace=ws)
    torch.cuda.synchronize()
    for k, (ws, outs, lses) in enumerate(bufs):
        for (r, T), o in outs.items():
            assert torch.equal(o, ref[T][0]) and torch.equal(lses[(r, T)], ref[T][1]), (k, r, T)


def test_write_then_attend_on_two_streams():
    """Each stream writes its own new rows into its own cache copy and then
    attends over lists that name those rows; the other stream does the same
    with other rows at the same slots."""
    print("writer + attention on two streams", flush=True)
    T = 100
    cfg = wl.config_rope_decode(T, seed=880, num_slots=32768, ctx=(2048, 32000))
    base = build_cache(cfg)
    q = bf16_dev(cfg["q"])
    idx_np = cfg["idx"]
    idx = torch.from_numpy(idx_np).to(DEV)
    valid = idx_np[idx_np > 0]
    rng = np.random.default_rng(881)
    new_slots = torch.from_numpy(rng.choice(np.unique(valid), size=T, replace=False).astype(np.int64)).to(DEV)
    lat = [bf16_dev(wl.normal_bf16(rng, (T, 512))) for _ in range(2)]
    pe = [bf16_dev(wl.normal_bf16(rng, (T, 64))) for _ in range(2)]

    ref = []
    for k in range(2):
        c = base.clone()
        smla.kv_write(lat[k], pe[k], new_slots, c)
        ref.append((c, smla.attn(q, c, idx, cfg["sm_scale"], 64)))
    torch.cuda.synchronize()
    assert not torch.equal(ref[0][1][0], ref[1][1][0])

    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    caches = [base.clone() for _ in range(2)]
    need = smla.workspace_size(T, 16, cfg["W"], 64)
    assert need > 0                      # two splits, merged in the launch
    ws = [torch.empty(need, dtype=torch.uint8, device=DEV) for _ in range(2)]
    outs = [[torch.empty((T, 16, 512), dtype=torch.bfloat16, device=DEV) for _ in range(REPS)]
            for _ in range(2)]
    lses = [[torch.empty((T, 16), dtype=torch.float32, device=DEV) for _ in range(REPS)] for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for r in range(REPS):
        for k, s in enumerate(streams):
            with torch.cuda.stream(s):
                smla.kv_write(lat[k], pe[k], new_slots, caches[k])
                smla.attn(q, caches[k], idx, cfg["sm_scale"], 64, out=outs[k][r], lse=lses[k][r], workspace=ws[k])
    torch.cuda.synchronize()
    for k in range(2):
        assert torch.equal(caches[k], ref[k][0]), k
        for r in range(REPS):
            assert torch.equal(outs[k][r], ref[k][1][0]) and torch.equal(lses[k][r], ref[k][1][1]), (k, r)


def test_results_do_not_depend_on_memory_load():
    """Every plan kind, the BF16 path, the gather and the writer give the same
    bits while another stream keeps HBM busy with large copies: latencies
    change, so a wait that were too short for its loads, or any other
    dependence on timing, would show."""
    print("calls under a background copy load", flush=True)
    cfg = wl.config_nope_decode(300, seed=890, num_slots=16384, ctx=(512, 16000))
    cache = build_cache(cfg)
    pf = wl.config_prefill(1024, seed=891, num_slots=8192)
    pcache = build_cache(pf)
    bcache = torch.zeros((cfg["num_slots"], 512), dtype=torch.bfloat16, device=DEV)
    smla.kv_write_bf16(bf16_dev(cfg["latent"]), None, torch.from_numpy(cfg["slots"]).to(DEV), bcache)
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(DEV)
    pq = bf16_dev(pf["q"])
    pidx = torch.from_numpy(pf["idx"]).to(DEV)
    rng = np.random.default_rng(892)
    gslots = torch.from_numpy(rng.integers(0, cfg["num_slots"], size=4096).astype(np.int64)).to(DEV)
    wlat = bf16_dev(wl.normal_bf16(rng, (512, 512)))
    wslots = torch.from_numpy(rng.choice(np.arange(1, cfg["num_slots"]), 512, replace=False).astype(np.int64)).to(DEV)
    torch.cuda.synchronize()

    def fp8(T):
        return lambda: smla.attn(q[:T].contiguous(), cache, idx[:T], cfg["sm_scale"], 0)

    def bf(T):
        return lambda: smla.attn_bf16(q[:T].contiguous(), bcache, idx[:T], cfg["sm_scale"])

    def write():
        c = cache.clone()
        smla.kv_write(wlat, None, wslots, c)
        return (c,)

    calls = [("fp8 T=%d" % T, fp8(T)) for T in (1, 16, 64, 100, 256, 300)]
    calls += [("bf16 T=%d" % T, bf(T)) for T in (16, 256)]
    calls += [("prefill 1024", lambda: smla.attn(pq, pcache, pidx, pf["sm_scale"], 64)),
              ("gather", lambda: (smla.gather_upconvert(cache, gslots, 0),)),
              ("writer", write)]
    quiet = {}
    for name, f in calls:
        quiet[name] = [t.clone() for t in f() if t is not None]
        torch.cuda.synchronize()

    src = torch.empty(256 << 20, dtype=torch.uint8, device=DEV)
    dst = torch.empty_like(src)
    bg = torch.cuda.Stream()
    bg.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = {}
        for name, f in calls:
            with torch.cuda.stream(bg):
                for _ in range(3):
                    dst.copy_(src)
            got[name] = f()
        torch.cuda.synchronize()
        for name, _ in calls:
            res = [t for t in got[name] if t is not None]
            assert all(torch.equal(a, b) for a, b in zip(res, quiet[name])), (rep, name)
