"""Benchmark of the sparse-MLA hot path on one MI355X.

A step is one pass of the whole path over one batch: mla_kv_write of the
batch's new KV rows, then sparse_mla_attn for the batch's query rows.  The
headline workload is GLM-style NoPE decode: 256 decode tokens, H=16, top-k
2048 in a buffer of width 2176, a 131,072-slot fp8_ds_mla cache of 64-token
pages, contexts U{1k..64k}.  `value` is algorithmic gathered KV bytes
(valid entries x 528 B) per step / step time, in GB/s.

Caches are rotated across steps (several copies whose total exceeds the
256 MB Infinity Cache), so each step's gathers come from HBM rather than a
cache left warm by the previous step.  The timed steps replay HIP graphs
captured from the library's launches (the library allocates nothing, so a
capture holds only the kernels): one graph runs a whole rotation, one step
per cache copy back to back, as a decode pass runs one layer after another,
and one more graph runs the steps left over when K is not a multiple of the
rotation.  That keeps host launch overhead out of the step time; each graph's
replay is checked bit for bit against eager steps.  Per-kernel durations come from HIP events
recorded on the library's stream around bursts of back-to-back launches.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
# Per-kernel bursts: BURST back-to-back launches after BURST_WARM untimed ones,
# queued behind a GPU-side sleep so that host launch pacing stays out.  A burst
# this short (~1 ms of attention) ends before the clock and power transient
# that a load step after an idle GPU shows 1.5-7 ms in; the rate it gives is
# the settled one.  The headline step timing (--warmup, --steps) runs its
# warm-up steps first and times the steps that follow, past that transient.
BURST, BURST_WARM = 20, 5
NOPE_ROW = 528      # bytes a NoPE reader gathers per entry
ROPE_ROW = 656


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=140)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-extras", action="store_true", help="headline step only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain device copies of 512 MiB (to scale HBM byte counters)")
    ap.add_argument("--case", default=None,
                    help="only time one attention workload (for profiling): " + ", ".join(CASES))
    return ap.parse_args()


# single attention workloads that --case runs alone: (generator, first T rows or None)
CASES = {
    "nope_decode_T256": ("nope", 256), "nope_decode_T64": ("nope", 64),
    "nope_decode_T16": ("nope", 16), "nope_decode_T1": ("nope", 1),
    "rope_decode_T256": ("rope", 256), "rope_decode_T64": ("rope", 64),
    "rope_decode_T16": ("rope", 16), "rope_decode_T1": ("rope", 1),
    "nope_decode_T512": ("nope", 512), "rope_decode_T512": ("rope", 512),
    "nope_disjoint_T256": ("disjoint_nope", 256), "rope_disjoint_T256": ("disjoint_rope", 256),
    "rope_disjoint_T64": ("disjoint64", 64),
    "prefill_T65": ("prefill", 65), "prefill_T128": ("prefill", 128), "prefill_T1024": ("prefill", 1024),
    # the gather alone (smla_gather_rows_probe) over the same rows
    "probe_nope_decode_T256": ("nope", 256), "probe_nope_disjoint_T256": ("disjoint_nope", 256),
    "probe_rope_disjoint_T256": ("disjoint_rope", 256),
}


def case_config(name):
    import workloads as wl
    kind, T = CASES[name]
    if kind == "nope":
        c = wl.config_nope_decode(64 if T < 256 else T)
    elif kind == "rope":
        c = wl.config_rope_decode(max(T, 256))
    elif kind == "disjoint_nope":
        return wl.config_disjoint_t256(0)
    elif kind == "disjoint_rope":
        return wl.config_disjoint_t256(64)
    elif kind == "disjoint64":
        return wl.config_disjoint(64)
    else:
        return wl.config_prefill(T)
    c = dict(c)
    c["q"], c["idx"] = c["q"][:T], c["idx"][:T]
    return c


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_nope_T256_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "sparse_mla_attention_fp8_amd", "csrc", "attn.hip")


def kernel_source_sha256() -> str:
    import hashlib
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of the headline attention kernel from the committed
    counter summary, or None when it is missing or was taken on other source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_sha256():
        return None
    return rec


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (got --gpus {a.gpus}); the "
              "multi-GPU sharding of the path is a design note, not a launchable mode.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if a.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "launches": 5}), flush=True)
        return
    import sparse_mla_attention_fp8_amd as smla
    import workloads as wl

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def build_cache(cfg):
        cache = torch.zeros((cfg["num_slots"], wl.ROW_BYTES), dtype=torch.uint8, device=dev)
        smla.kv_write(bf16_dev(cfg["latent"]),
                      bf16_dev(cfg["rope"]) if cfg["rope"] is not None else None,
                      torch.from_numpy(cfg["slots"]).to(dev), cache)
        cache[0] = torch.from_numpy(cfg["slot0"]).to(dev)
        torch.cuda.synchronize()
        return cache

    def rotations(cache):
        n = max(2, int(np.ceil(600e6 / cache.numel())))   # > 2x the Infinity Cache
        return [cache] + [cache.clone() for _ in range(n - 1)]

    def burst(launch, iters, warm):
        """Average duration (us) of `iters` back-to-back launches between one
        pair of events on the library's stream, after `warm` untimed ones."""
        for i in range(warm):
            launch(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # a fixed-length GPU delay first, so that every launch of the burst is
        # queued before the first one starts (host launch pacing stays out)
        torch.cuda._sleep(int(2.0e6 + 150e3 * iters))
        e0.record(stream)
        for i in range(iters):
            launch(warm + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) * 1e3 / iters])

    def time_attn(cfg, caches, iters, warm):
        q = bf16_dev(cfg["q"])
        idx = torch.from_numpy(cfg["idx"]).to(dev)
        W = cfg["idx"].shape[1]
        T, H = q.shape[0], q.shape[1]
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws_n = smla.workspace_size(T, H, W, cfg["rope_dim"])
        ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
        def launch(i):
            smla.attn(q, caches[i % len(caches)], idx, cfg["sm_scale"], cfg["rope_dim"],
                      topk_capacity=W, out=out, lse=lse, workspace=ws)
        return burst(launch, iters, warm), out, lse

    def gathered(cfg, row_bytes):
        idx = cfg["idx"]
        return int(((idx >= 0) & (idx < cfg["num_slots"])).sum()) * row_bytes

    def valid_list(cfg):
        v = cfg["idx"].ravel()
        return torch.from_numpy(np.ascontiguousarray(v[(v >= 0) & (v < cfg["num_slots"])])).to(dev)

    def time_probe(cfg, caches, iters, warm):
        """The gather alone over the call's valid entries (the attention's rows)."""
        sl = valid_list(cfg)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        return burst(lambda i: smla.gather_rows_probe(caches[i % len(caches)], sl, cfg["rope_dim"], sink),
                     iters, warm)

    if a.case is not None:
        log(f"case {a.case}")
        c = case_config(a.case)
        cache = build_cache(c)
        rot = [cache] if a.case.startswith("prefill") else rotations(cache)
        if a.case.startswith("probe_"):
            us = time_probe(c, rot, a.steps, a.warmup)
        else:
            us, _, _ = time_attn(c, rot, a.steps, a.warmup)
        b = gathered(c, ROPE_ROW if c["rope_dim"] else NOPE_ROW)
        print(json.dumps({"case": a.case, "us": round(float(us.mean()), 2),
                          "gathered_bytes": b, "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1),
                          "launches": a.steps + a.warmup}), flush=True)
        return

    # ---------------- headline: NoPE decode T=256, writer + attention ---------------
    T = 256
    log("generating NoPE decode workload (T=256, 131072 slots)")
    cfg = wl.config_nope_decode(T)
    cache0 = build_cache(cfg)
    caches = rotations(cache0)
    rng = np.random.default_rng(99)
    new_lat = bf16_dev(wl.normal_bf16(rng, (T, 512)))
    new_slots = torch.from_numpy(rng.choice(cfg["num_slots"] - 1, T, replace=False).astype(np.int64) + 1).to(dev)
    q = bf16_dev(cfg["q"])
    idx = torch.from_numpy(cfg["idx"]).to(dev)
    W = cfg["idx"].shape[1]
    out = torch.empty((T, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, 16), dtype=torch.float32, device=dev)
    ws_n = smla.workspace_size(T, 16, W, 0)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    bytes_step = gathered(cfg, NOPE_ROW)

    def step(i):
        c = caches[i % len(caches)]
        smla.kv_write(new_lat, None, new_slots, c)
        smla.attn(q, c, idx, cfg["sm_scale"], 0, topk_capacity=W, out=out, lse=lse, workspace=ws)

    # The timed steps run as graphs of up to one rotation each (steps
    # W + 7j .. W + 7j + 6 share one graph, as their cache copies repeat) plus
    # one graph for the last K mod 7 steps; eager launches if capture is
    # unavailable.
    launch_mode = "hip-graph"
    rot = len(caches)
    full = tail = None
    n_full, n_tail = a.steps // rot, a.steps % rot

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + count):
                step(i)
        return g

    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(rot):
                step(k)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = out.clone()
        if n_full:
            full = capture(a.warmup, rot)
        if n_tail:
            tail = capture(a.warmup + n_full * rot, n_tail)
        for g in (full, tail):
            if g is None:
                continue
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError("graph replay differs from the eager steps")
    except Exception as exc:   # noqa: BLE001 - report and fall back to eager launches
        log(f"graph capture unavailable ({exc}); timing eager launches")
        full = tail = None
        launch_mode = "eager"

    for i in range(a.warmup):
        step(i)
    log(f"timing {a.steps} steps ({launch_mode})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if launch_mode == "hip-graph":
        for _ in range(n_full):
            full.replay()
        if tail is not None:
            tail.replay()
    else:
        for i in range(a.steps):
            step(a.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / a.steps
    del full, tail
    # per-kernel durations: bursts of back-to-back launches, caches rotated
    attn_us = burst(lambda i: smla.attn(q, caches[i % len(caches)], idx, cfg["sm_scale"], 0,
                                        topk_capacity=W, out=out, lse=lse, workspace=ws),
                    BURST, BURST_WARM)
    # warm: the same cache copy every launch, so rows the previous launch
    # gathered may still sit in the Infinity Cache
    attn_warm = burst(lambda i: smla.attn(q, caches[0], idx, cfg["sm_scale"], 0, topk_capacity=W,
                                          out=out, lse=lse, workspace=ws), BURST, BURST_WARM)
    wr_us = burst(lambda i: smla.kv_write(new_lat, None, new_slots, caches[i % len(caches)]),
                  BURST, BURST_WARM)
    probe_us = time_probe(cfg, caches, BURST, BURST_WARM)
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    attn_gbs = bytes_step / (attn_us.mean() * 1e-6) / 1e9
    log(f"step {ms_per_step*1e3:.1f} us, attention {attn_us.mean():.1f} us "
        f"({attn_gbs:.0f} GB/s), writer {wr_us.mean():.2f} us")

    result = {
        "metric": "sparse-MLA decode KV GB/s + % HBM peak (H=16, topk 2048); KV-writer rows/us",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded N(0,1) bf16 rows, fp8_ds_mla cache written by mla_kv_write)",
        "config": {
            "workload": "GLM-style NoPE sparse-MLA decode: 256 tokens, H=16, top-k 2048 in a "
                        "2176-wide buffer, 131072-slot fp8_ds_mla cache of 64-token pages, "
                        "contexts U{1k..64k}, slot 0 = 0x7F; step = mla_kv_write(256 rows) + "
                        "sparse_mla_attn",
            "batch": T, "heads": 16, "topk": 2048, "topk_width": W, "rope_dim": 0,
            "num_slots": cfg["num_slots"], "cache_rotation": len(caches),
            "launch": launch_mode,
        },
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "attn_us": round(float(attn_us.mean()), 2),
        "attn_gbs": round(attn_gbs, 1),
        "attn_hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4),
        "attn_warm_us": round(float(attn_warm.mean()), 2),
        "gather_only_us": round(float(probe_us.mean()), 2),
        "attn_over_gather_only": round(float(probe_us.mean() / attn_us.mean()), 4),
        "writer_step_us": round(float(wr_us.mean()), 3),
        "gathered_bytes_per_step": bytes_step,
        "unique_row_bytes_per_step": int(np.unique(cfg["idx"][cfg["idx"] >= 0]).size) * NOPE_ROW,
    }
    # the three byte counts side by side, each over the attention launch's time:
    # algorithmic (attn_gbs), distinct rows only, and counter-derived (below)
    result["attn_unique_row_gbs"] = round(result["unique_row_bytes_per_step"] / (attn_us.mean() * 1e3), 1)
    result["roofline"] = {
        "bound": "hbm",
        "achieved": round(attn_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
        "traffic": None,
        "kernel": "sparse_mla_attn main kernel, NoPE T=256 (one split per row, no merge)",
    }
    tr = measured_traffic()
    if tr is not None:
        result["roofline"]["traffic"] = tr["hbm_bytes_per_launch"]
        result["attn_counter_gbs"] = round(tr["hbm_bytes_per_launch"] / (attn_us.mean() * 1e3), 1)
        result["roofline"]["traffic_detail"] = {k: tr[k] for k in
                                                ("fetch_bytes_per_launch", "write_bytes_per_launch",
                                                 "copy_scale_fetch", "copy_scale_write")}
    del caches

    extras = {}

    def gather_extra(name, rot, rope_dim, n=65536):
        """mla_gather_upconvert of n distinct random slots into bf16 [n][576],
        cache copies rotated; algorithmic bytes: slot ids, the row bytes read
        (528 or 656) and the 1,152 bytes written per row."""
        num_slots = rot[0].shape[0]
        rng_g = np.random.default_rng(80 + rope_dim)
        sl = torch.from_numpy(rng_g.choice(np.arange(1, num_slots), size=n, replace=False)
                              .astype(np.int64)).to(dev)
        dst = torch.empty((n, 576), dtype=torch.bfloat16, device=dev)
        us = burst(lambda i: smla.gather_upconvert(rot[i % len(rot)], sl, rope_dim, out=dst),
                   BURST, BURST_WARM)
        byts = n * (8 + (ROPE_ROW if rope_dim else NOPE_ROW) + 1152)
        extras[name] = {"us": round(float(us.mean()), 2),
                        "gbs": round(byts / (us.mean() * 1e-6) / 1e9, 1),
                        "hbm_frac": round(byts / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"{name}: {us.mean():.2f} us")

    if not a.no_extras:
        # writer standalone: 8,192 rows, a quarter aimed at slot 0 with NaN inputs
        for N in (8192, 1024):
            for rope_dim in (64, 0):
                wc = wl.config_writer(N=N, rope_dim=rope_dim)
                cache = torch.from_numpy(wc["cache"]).to(dev)
                lat = bf16_dev(wc["latent"])
                rope = bf16_dev(wc["rope"]) if rope_dim else None
                sl = torch.from_numpy(wc["slots"]).to(dev)
                us = burst(lambda i: smla.kv_write(lat, rope, sl, cache), BURST, BURST_WARM)
                written = int((wc["slots"] > 0).sum())
                byts = written * ((1024 + (128 if rope_dim else 0)) + 656 + 8) + (N - written) * 8
                extras[f"writer_{N}_rope{rope_dim}"] = {
                    "us": round(float(us.mean()), 3),
                    "rows_per_us": round(N / us.mean(), 1),
                    "written_rows_per_us": round(written / us.mean(), 1),
                    "gbs": round(byts / (us.mean() * 1e-6) / 1e9, 1),
                }
                log(f"writer {N} rope{rope_dim}: {us.mean():.2f} us")
        # NoPE decode curve
        cfgc = wl.config_nope_decode(64)
        cachec = build_cache(cfgc)
        rot = rotations(cachec)
        for Tc in (1, 16, 64):
            sub = dict(cfgc)
            sub["q"], sub["idx"] = cfgc["q"][:Tc], cfgc["idx"][:Tc]
            us, _, _ = time_attn(sub, rot, BURST, BURST_WARM)
            b = gathered(sub, NOPE_ROW)
            extras[f"nope_decode_T{Tc}"] = {"us": round(float(us.mean()), 2),
                                           "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1)}
            log(f"nope T={Tc}: {us.mean():.1f} us")
        gather_extra("gather_upconvert_nope_N65536", rot, 0)
        del rot, cachec
        # the no-reuse controls: the headline batch shape with pairwise disjoint
        # top-k sets on a 1,048,576-slot cache, so gathered bytes are unique
        # bytes and every gathered row is read once per launch (NoPE in the
        # 2176-wide buffer, RoPE in a 2048-wide one)
        for name, rope_dim in (("nope_disjoint_T256", 0), ("rope_disjoint_T256", 64)):
            log(f"generating {name}")
            c = wl.config_disjoint_t256(rope_dim)
            cache = build_cache(c)
            rot = rotations(cache)
            us, _, _ = time_attn(c, rot, BURST, BURST_WARM)
            pus = time_probe(c, rot, BURST, BURST_WARM)
            b = gathered(c, ROPE_ROW if rope_dim else NOPE_ROW)
            extras[name] = {"us": round(float(us.mean()), 2),
                            "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1),
                            "hbm_frac": round(b / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "gathered_bytes": b, "unique_row_bytes": b,
                            "gather_only_us": round(float(pus.mean()), 2),
                            "gather_only_hbm_frac": round(b / (pus.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "attn_over_gather_only": round(float(pus.mean() / us.mean()), 4)}
            log(f"{name}: {us.mean():.1f} us")
            del rot, cache, c
        # RoPE decode T=256 and the smaller disjoint control
        for name, c in (("rope_decode_T256", wl.config_rope_decode(256)),
                        ("rope_disjoint_T64", wl.config_disjoint(64))):
            log(f"generating {name}")
            cache = build_cache(c)
            rot = rotations(cache)
            us, _, _ = time_attn(c, rot, BURST, BURST_WARM)
            b = gathered(c, ROPE_ROW)
            extras[name] = {"us": round(float(us.mean()), 2),
                            "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1),
                            "hbm_frac": round(b / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"{name}: {us.mean():.1f} us")
            if name == "rope_decode_T256":
                gather_extra("gather_upconvert_rope_N65536", rot, 64)
                # the RoPE decode curve: the first T rows of the same batch
                for Tc in (1, 16, 64):
                    sub = dict(c)
                    sub["q"], sub["idx"] = c["q"][:Tc], c["idx"][:Tc]
                    us, _, _ = time_attn(sub, rot, BURST, BURST_WARM)
                    b = gathered(sub, ROPE_ROW)
                    extras[f"rope_decode_T{Tc}"] = {"us": round(float(us.mean()), 2),
                                                   "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1)}
                    log(f"rope T={Tc}: {us.mean():.1f} us")
            del rot, cache
        # sparse prefill of one causal sequence (rope 64): row t attends over
        # tokens 0..t, so the rows are re-read from L2 and the kernel is not
        # HBM-bound; reported as algorithmic score + P.V FLOP/s
        for Tp in (65, 128, 1024):
            cp = wl.config_prefill(Tp)
            cache = build_cache(cp)
            us, _, _ = time_attn(cp, [cache], BURST, BURST_WARM)
            nv = int((cp["idx"] >= 0).sum())
            flops = 2.0 * 16 * (576 + 512) * nv
            extras[f"prefill_T{Tp}"] = {"us": round(float(us.mean()), 2),
                                        "tflops": round(flops / (us.mean() * 1e-6) / 1e12, 2),
                                        "query_rows_per_us": round(Tp / us.mean(), 3)}
            log(f"prefill T={Tp}: {us.mean():.1f} us")
            del cache
        # BF16 KV cache: NoPE decode T=256 over rows of 512 bf16 values
        cb = wl.config_nope_decode(256)
        log("generating bf16_nope_decode_T256")
        cacheb = torch.zeros((cb["num_slots"], 512), dtype=torch.bfloat16, device=dev)
        smla.kv_write_bf16(bf16_dev(cb["latent"]), None, torch.from_numpy(cb["slots"]).to(dev), cacheb)
        nrb = max(2, int(np.ceil(600e6 / (cacheb.numel() * 2))))
        rotb = [cacheb] + [cacheb.clone() for _ in range(nrb - 1)]
        qb_ = bf16_dev(cb["q"])
        idxb = torch.from_numpy(cb["idx"]).to(dev)
        ob = torch.empty((256, 16, 512), dtype=torch.bfloat16, device=dev)
        lb = torch.empty((256, 16), dtype=torch.float32, device=dev)
        us = burst(lambda i: smla.attn_bf16(qb_, rotb[i % nrb], idxb, cb["sm_scale"], out=ob, lse=lb),
                   BURST, BURST_WARM)
        b = gathered(cb, 1024)
        extras["bf16_nope_decode_T256"] = {"us": round(float(us.mean()), 2),
                                           "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1),
                                           "hbm_frac": round(b / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"bf16_nope_decode_T256: {us.mean():.1f} us")
        del rotb, cacheb
        # BF16 KV cache: RoPE decode T=256 over rows of 512 + 64 bf16 values
        cr = wl.config_rope_decode(256)
        log("generating bf16_rope_decode_T256")
        cacher = torch.zeros((cr["num_slots"], 576), dtype=torch.bfloat16, device=dev)
        smla.kv_write_bf16(bf16_dev(cr["latent"]), bf16_dev(cr["rope"]),
                           torch.from_numpy(cr["slots"]).to(dev), cacher)
        nrr = max(2, int(np.ceil(600e6 / (cacher.numel() * 2))))
        rotr = [cacher] + [cacher.clone() for _ in range(nrr - 1)]
        qr_ = bf16_dev(cr["q"])
        idxr = torch.from_numpy(cr["idx"]).to(dev)
        us = burst(lambda i: smla.attn_bf16(qr_, rotr[i % nrr], idxr, cr["sm_scale"], out=ob, lse=lb),
                   BURST, BURST_WARM)
        b = gathered(cr, 1152)
        extras["bf16_rope_decode_T256"] = {"us": round(float(us.mean()), 2),
                                           "gbs": round(b / (us.mean() * 1e-6) / 1e9, 1),
                                           "hbm_frac": round(b / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"bf16_rope_decode_T256: {us.mean():.1f} us")
        del rotr, cacher
        wb = wl.config_writer(N=8192, rope_dim=0)
        wcache = torch.zeros((wb["cache"].shape[0], 512), dtype=torch.bfloat16, device=dev)
        wlat = bf16_dev(wb["latent"])
        wsl = torch.from_numpy(wb["slots"]).to(dev)
        us = burst(lambda i: smla.kv_write_bf16(wlat, None, wsl, wcache), BURST, BURST_WARM)
        written = int((wb["slots"] > 0).sum())
        extras["writer_bf16_8192_rope0"] = {"us": round(float(us.mean()), 3),
                                            "rows_per_us": round(8192 / us.mean(), 1),
                                            "gbs": round((written * (1024 + 1024 + 8) + (8192 - written) * 8)
                                                         / (us.mean() * 1e-6) / 1e9, 1)}
        log(f"writer bf16 rope0: {us.mean():.2f} us")
        del wcache
        # LSE merge of 8 partial results (context-parallel decode over 8 owners),
        # T=256, H=16; inputs rotated over copies larger than the Infinity Cache
        Pm, Tm, Hm = 8, 256, 16
        rng_m = np.random.default_rng(70)
        po = bf16_dev(wl.normal_bf16(rng_m, (Pm, Tm, Hm, 512)))
        pl = torch.from_numpy(rng_m.uniform(-8, 8, size=(Pm, Tm, Hm)).astype(np.float32)).to(dev)
        nrot = max(2, int(np.ceil(600e6 / (po.numel() * 2))))
        pos = [po] + [po.clone() for _ in range(nrot - 1)]
        mo = torch.empty((Tm, Hm, 512), dtype=torch.bfloat16, device=dev)
        ml = torch.empty((Tm, Hm), dtype=torch.float32, device=dev)
        us = burst(lambda i: smla.merge(pos[i % nrot], pl, out=mo, lse=ml), BURST, BURST_WARM)
        byts = (Pm + 1) * Tm * Hm * (1024 + 4)
        extras["merge_P8_T256"] = {"us": round(float(us.mean()), 2),
                                   "gbs": round(byts / (us.mean() * 1e-6) / 1e9, 1),
                                   "hbm_frac": round(byts / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"merge P=8 T=256: {us.mean():.2f} us")
        del pos, po
        # page re-split: all 512 pages of a 131,072-slot pool of 256-token pages
        # into a 64-token scratch (a step that touches every page)
        npg = 512
        pools = [torch.zeros((npg, 256 * wl.ROW_BYTES), dtype=torch.uint8, device=dev) for _ in range(4)]
        scratch = torch.zeros((4 * npg, 64 * wl.ROW_BYTES), dtype=torch.uint8, device=dev)
        pg = torch.arange(npg, dtype=torch.int32, device=dev)
        us = burst(lambda i: smla.split_pages_64(pools[i % 4], pg, scratch), BURST, BURST_WARM)
        byts = 2 * npg * 256 * wl.ROW_BYTES + 4 * npg
        extras["split_pages_512x256"] = {"us": round(float(us.mean()), 2),
                                         "gbs": round(byts / (us.mean() * 1e-6) / 1e9, 1),
                                         "hbm_frac": round(byts / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"split pages 512 x 256: {us.mean():.2f} us")
        del pools, scratch
    result["extras"] = extras

    # ---------------- oracle on the host cores, bounded sample ----------------
    if not a.no_cpu:
        from threadpoolctl import threadpool_limits
        from oracle import attention as oattn
        from oracle import writer as owriter
        # the host cores this process may run on, capped by the thread budget
        # the environment grants (OMP_NUM_THREADS), which BLAS would use anyway
        cores = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():
            cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
        need = cfg["idx"].ravel()
        need = np.unique(need[need >= 0])
        ocache = np.zeros((cfg["num_slots"], wl.ROW_BYTES), dtype=np.uint8)
        ocache[need] = owriter.encode_rows(cfg["latent"][need - 1], None)

        def time_oracle_attn(threads, budget):
            passes, dt = 0, 0.0
            with threadpool_limits(limits=threads):
                while dt < budget and passes < 50:
                    t0 = time.perf_counter()
                    oattn.sparse_mla_attn(cfg["q"], ocache, cfg["idx"], W, 0, cfg["sm_scale"])
                    dt += time.perf_counter() - t0
                    passes += 1
            return passes, dt

        def time_oracle_writer(wc, threads, budget):
            passes, dt = 0, 0.0
            with threadpool_limits(limits=threads):
                while dt < budget and passes < 50:
                    wcache = wc["cache"].copy()
                    t0 = time.perf_counter()
                    owriter.kv_write(wcache, wc["latent"], wc["rope"], wc["slots"])
                    dt += time.perf_counter() - t0
                    passes += 1
            return passes, dt

        passes, dt = time_oracle_attn(cores, 10.0)           # about 10 s of host work
        result["cpu_baseline"] = {
            "value": round(bytes_step * passes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"float64 numpy oracle attention over the whole 256-row NoPE decode batch, "
                      f"{passes} passes in {dt:.1f} s, BLAS threads = {cores} (the host cores "
                      f"this process may use)",
        }
        log(f"oracle ({cores} threads): {dt:.2f} s for {passes} passes")
        p1, dt1 = time_oracle_attn(1, 5.0)
        result["cpu_baseline_1thread"] = {
            "value": round(bytes_step * p1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the same oracle attention, BLAS pinned to 1 thread, {p1} passes in {dt1:.1f} s",
        }
        log(f"oracle (1 thread): {dt1:.2f} s for {p1} passes")
        # the writer half of the metric: the oracle writer on the 8,192-row call
        wc = wl.config_writer(N=8192, rope_dim=64)
        for key, threads, budget in (("cpu_baseline_writer", cores, 3.0),
                                     ("cpu_baseline_writer_1thread", 1, 2.0)):
            wp, wdt = time_oracle_writer(wc, threads, budget)
            result[key] = {
                "value": round(8192 * wp / (wdt * 1e6), 3), "unit": "rows/us", "cores": threads,
                "kind": "oracle",
                "sample": f"float64 numpy oracle writer on the 8,192-row call (rope 64, a quarter "
                          f"padding rows), {wp} passes in {wdt:.1f} s, BLAS threads = {threads}",
            }
            log(f"oracle writer ({threads} threads): {wdt:.2f} s for {wp} passes")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    main()
