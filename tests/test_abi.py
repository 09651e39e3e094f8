"""The C-ABI library loads, exports every entry point of include/*.h, and
rejects bad arguments on the host before any GPU work (no device needed)."""
import ctypes
import glob
import os
import re
import subprocess
import sys

import pytest

import sparse_mla_attention_fp8_amd as smla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:SMLA_API\s+)?(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"mla_kv_write", "sparse_mla_attn", "sparse_mla_attn_workspace_size",
            "smla_last_error"} <= names
    raw = ctypes.CDLL(smla.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(smla._SIGS) == names


def test_only_the_declared_entry_points_are_exported():
    """The library's internal C++ symbols stay hidden (built with hidden
    visibility; the headers mark the entry points for export)."""
    names = _declared()
    out = subprocess.run(["nm", "-D", "--defined-only", smla.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    functions = {line.split()[-1] for line in out.splitlines() if len(line.split()) == 3 and line.split()[1] == "T"}
    assert functions == names, sorted(functions ^ names)


FAKE = 0x10000          # an aligned address that is never dereferenced


def test_kv_write_validation():
    L = smla.lib()
    bad = [
        dict(rope_dim=5),
        dict(kv_c=None),
        dict(slot_mapping=None),
        dict(kv_cache=None),
        dict(k_pe=None),                      # rope_dim 64 needs k_pe
        dict(rope_dim=0),                     # k_pe must be NULL with rope 0
        dict(kv_c_row_stride=500),
        dict(kv_c_row_stride=516),
        dict(k_pe_row_stride=60),
        dict(kv_c=FAKE + 8),
        dict(num_rows=-1),
        dict(num_slots=0),
    ]
    base = dict(kv_c=FAKE, kv_c_row_stride=512, k_pe=FAKE, k_pe_row_stride=64, rope_dim=64,
                slot_mapping=FAKE, num_rows=4, kv_cache=FAKE, num_slots=128, stream=None)
    for b in bad:
        a = {**base, **b}
        rc = L.mla_kv_write(*a.values())
        assert rc == smla.SMLA_EINVAL, b
        assert L.smla_last_error().decode().startswith("mla_kv_write")
    # zero rows is a no-op that launches nothing
    assert L.mla_kv_write(*{**base, "num_rows": 0}.values()) == smla.SMLA_OK
    # a row count whose grid would not fit is refused before any launch
    assert L.mla_kv_write(*{**base, "num_rows": 1 << 34}.values()) == smla.SMLA_EUNSUPPORTED
    assert L.mla_kv_write_bf16(*{**base, "num_rows": 1 << 34}.values()) == smla.SMLA_EUNSUPPORTED


def test_attn_validation():
    L = smla.lib()
    base = dict(q=FAKE, kv_cache=FAKE, num_slots=4096, topk_idx=FAKE, idx_row_stride=2176,
                topk_capacity=2176, T=4, H=16, rope_dim=0, sm_scale=0.04, out=FAKE, lse=None,
                workspace=None, workspace_bytes=0, stream=None)
    bad = [
        (dict(rope_dim=32), smla.SMLA_EINVAL),
        (dict(T=0), smla.SMLA_EINVAL),
        (dict(H=0), smla.SMLA_EINVAL),
        (dict(H=129), smla.SMLA_EINVAL),
        (dict(topk_capacity=0), smla.SMLA_EINVAL),
        (dict(idx_row_stride=2048), smla.SMLA_EINVAL),
        (dict(num_slots=0), smla.SMLA_EINVAL),
        (dict(q=None), smla.SMLA_EINVAL),
        (dict(out=None), smla.SMLA_EINVAL),
        (dict(q=FAKE + 4), smla.SMLA_EINVAL),
        (dict(sm_scale=float("nan")), smla.SMLA_EINVAL),
        (dict(T=70000), smla.SMLA_EUNSUPPORTED),
        (dict(T=4), smla.SMLA_EWORKSPACE),    # 4 rows need split partials
        (dict(T=4, workspace=FAKE, workspace_bytes=16), smla.SMLA_EWORKSPACE),
    ]
    for b, code in bad:
        a = {**base, **b}
        rc = L.sparse_mla_attn(*a.values())
        assert rc == code, (b, rc)
        assert L.smla_last_error().decode().startswith("sparse_mla_attn")


def test_workspace_size():
    assert smla.workspace_size(0, 16, 2048, 64) == 0
    assert smla.workspace_size(4, 16, 2048, 77) == 0
    big = smla.workspace_size(256, 16, 2048, 64)
    small = smla.workspace_size(1, 16, 2048, 64)
    assert small > 0
    # one split per row needs no partials; whatever is returned is a whole number of
    # fp32 [H][514] records per (row, split)
    for T in (1, 2, 16, 64, 256):
        ws = smla.workspace_size(T, 16, 2176, 0)
        assert ws % (16 * 514 * 4 * T) == 0
    assert big % (16 * 514 * 4 * 256) == 0


def test_merge_validation():
    L = smla.lib()
    base = dict(part_out=FAKE, part_lse=FAKE, P=2, T=3, H=16, out=FAKE + 0x100000, lse=None, stream=None)
    bad = [
        dict(P=0), dict(T=0), dict(H=0), dict(H=129),
        dict(part_out=None), dict(part_lse=None), dict(out=None),
        dict(part_out=FAKE + 8), dict(out=FAKE + 0x100008), dict(part_lse=FAKE + 2), dict(lse=FAKE + 2),
    ]
    for b in bad:
        a = {**base, **b}
        rc = L.sparse_mla_merge(*a.values())
        assert rc == smla.SMLA_EINVAL, b
        assert L.smla_last_error().decode().startswith("sparse_mla_merge")


def test_gather_validation():
    L = smla.lib()
    base = dict(kv_cache=FAKE, num_slots=128, rope_dim=64, slots=FAKE, num_rows=4,
                dst=FAKE + 0x100000, dst_row_stride=576, stream=None)
    bad = [
        dict(rope_dim=32), dict(num_rows=-1), dict(num_slots=0),
        dict(kv_cache=None), dict(slots=None), dict(dst=None),
        dict(dst_row_stride=512), dict(dst_row_stride=580),
        dict(kv_cache=FAKE + 8), dict(dst=FAKE + 0x100008), dict(slots=FAKE + 4),
    ]
    for b in bad:
        a = {**base, **b}
        rc = L.mla_gather_upconvert(*a.values())
        assert rc == smla.SMLA_EINVAL, b
        assert L.smla_last_error().decode().startswith("mla_gather_upconvert")
    assert L.mla_gather_upconvert(*{**base, "num_rows": 0, "kv_cache": None}.values()) in (smla.SMLA_OK, smla.SMLA_EINVAL)


def test_split_pages_validation():
    L = smla.lib()
    base = dict(src=FAKE, num_src=8, src_stride=256 * 656, pages=FAKE, num_pages=4,
                dst=FAKE + 0x1000000, dst_stride=64 * 656, row_bytes=656, stream=None)
    bad = [
        dict(row_bytes=0), dict(row_bytes=-16), dict(num_src=0), dict(num_pages=-1),
        dict(src=None), dict(pages=None), dict(dst=None),
        dict(src_stride=256 * 656 - 16), dict(dst_stride=64 * 656 - 16), dict(dst_stride=64 * 656 + 8),
        dict(src=FAKE + 8), dict(pages=FAKE + 2),
    ]
    for b in bad:
        a = {**base, **b}
        rc = L.mla_split_pages_64(*a.values())
        assert rc == smla.SMLA_EINVAL, b
        assert L.smla_last_error().decode().startswith("mla_split_pages_64")


def test_plan_fits_one_round_of_workgroups():
    """One workgroup runs per CU (256 on the chip), so the split count keeps a
    launch to one round of workgroups: 65 rows take 3 splits (195 workgroups),
    not 4 (260, where 4 would wait for a second round).  Plans of two or three
    splits merge inside the launch and add one 8-byte arrival word per
    (row, head group) to the partials."""
    rec = 16 * 514 * 4
    for T in range(1, 300):
        ws = smla.workspace_size(T, 16, 2048, 64)
        s = ws // (rec * T) if ws else 1
        words = 8 * T if 2 <= s <= 3 else 0
        assert ws == 0 or ws == s * rec * T + words
        assert s == 1 or s * T <= 256, (T, s)
        # no more splits than chunks: 64-key chunks, or 32-key ones for a single row
        assert s <= (64 if T == 1 else 32)
    assert smla.workspace_size(65, 16, 2048, 64) == 3 * rec * 65 + 8 * 65
    assert smla.workspace_size(100, 16, 2176, 0) == 2 * rec * 100 + 8 * 100
    assert smla.workspace_size(40, 32, 2176, 0) == 3 * (2 * rec) * 40 + 8 * 40 * 2
    assert smla.workspace_size(64, 16, 2176, 0) == 4 * rec * 64
    assert smla.workspace_size(257, 16, 2048, 64) == 0


def test_missing_library_raises(monkeypatch):
    """No fallback: without the built library every entry point raises."""
    monkeypatch.setattr(smla, "_lib", None)
    monkeypatch.setattr(smla, "LIB_PATH", os.path.join(os.path.dirname(smla.LIB_PATH), "absent.so"))
    with pytest.raises(ImportError):
        smla.lib()
    with pytest.raises(ImportError):
        smla.workspace_size(1, 16, 2048, 64)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asking for more exits with a message."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


# ---- the Python binding refuses mismatched tensors before any launch ----------
# Shape and dtype checks run before the device check, so host tensors exercise
# them here; a host tensor with correct shapes is refused by the device check.

def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def _raises(fn, *args, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_binding_kv_write_checks():
    import torch
    n = 8
    kv_c, k_pe = _bf(n, 512), _bf(n, 64)
    slots = torch.arange(1, n + 1, dtype=torch.int64)
    cache = torch.zeros((64, 656), dtype=torch.uint8)
    _raises(smla.kv_write, _bf(n, 500), None, slots, cache, match="kv_c rows must hold")
    _raises(smla.kv_write, kv_c, None, slots[:5], cache, match="slot_mapping has 5 entries")
    _raises(smla.kv_write, kv_c, None, slots.int(), cache, match="int64")
    _raises(smla.kv_write, kv_c, _bf(n - 1, 64), slots, cache, match="k_pe has 7 rows")
    _raises(smla.kv_write, kv_c, _bf(n, 32), slots, cache, match="k_pe rows must hold >= 64")
    _raises(smla.kv_write, kv_c, k_pe, slots, torch.zeros((64, 528), dtype=torch.uint8), match="kv_cache")
    _raises(smla.kv_write, kv_c, k_pe, slots, cache.view(8, 8, 656), match="kv_cache")
    _raises(smla.kv_write, kv_c, k_pe, slots, cache, match="must be a GPU tensor")
    _raises(smla.kv_write_bf16, kv_c, None, slots[:3], _bf(64, 512), match="slot_mapping has 3")
    _raises(smla.kv_write_bf16, kv_c, k_pe, slots, _bf(64, 512), match=r"\[num_slots\]\[576\]")
    _raises(smla.kv_write_bf16, kv_c, k_pe, slots, _bf(64, 576), match="must be a GPU tensor")


def test_binding_attn_checks():
    import torch
    T, H = 4, 16
    q = _bf(T, H, 512)
    cache = torch.zeros((128, 656), dtype=torch.uint8)
    idx = torch.full((T, 2176), -1, dtype=torch.int32)
    _raises(smla.attn, q, cache, idx, 0.04, 64, match="q rows are 512 wide")
    _raises(smla.attn, q, cache, idx, 0.04, 32, match="rope_dim must be 0 or 64")
    _raises(smla.attn, q, cache, idx[:3], 0.04, 0, match="topk_idx has 3 rows for 4")
    _raises(smla.attn, q, cache, idx, 0.04, 0, topk_capacity=2200, match="topk_capacity 2200")
    _raises(smla.attn, q, cache, idx, 0.04, 0, topk_capacity=0, match="topk_capacity 0")
    _raises(smla.attn, q, cache, idx.long(), 0.04, 0, match="int32")
    _raises(smla.attn, q, cache[:, :528], idx, 0.04, 0, match="kv_cache")
    _raises(smla.attn, q, cache, idx, 0.04, 0, out=_bf(T, H, 576), match="out must be")
    _raises(smla.attn, q, cache, idx, 0.04, 0, lse=torch.zeros((T, H + 1)), match="lse must be")
    _raises(smla.attn, q, cache, idx, 0.04, 0, match="q must be a GPU tensor")
    _raises(smla.attn_bf16, q, _bf(128, 576), idx, 0.04, match=r"\[num_slots\]\[512\]")
    _raises(smla.attn_bf16, _bf(T, H, 600), _bf(128, 600), idx, 0.04, match="512 or 576 wide")
    _raises(smla.attn_bf16, q, _bf(128, 512), idx[:, :0], 0.04, match="topk_capacity 0")
    _raises(smla.attn_bf16, q, _bf(128, 512), idx, 0.04, match="q must be a GPU tensor")


def test_binding_other_checks():
    import torch
    cache = torch.zeros((128, 656), dtype=torch.uint8)
    slots = torch.arange(4, dtype=torch.int64)
    _raises(smla.gather_upconvert, cache, slots, 16, match="rope_dim")
    _raises(smla.gather_upconvert, cache, slots, 0, out=_bf(3, 576), match="out has 3 rows for 4")
    _raises(smla.gather_upconvert, cache, slots, 0, out=_bf(4, 512), match="out rows must hold >= 576")
    _raises(smla.gather_upconvert, cache, slots, 0, match="must be a GPU tensor")
    po, pl = _bf(2, 3, 16, 512), torch.zeros((2, 3, 16))
    _raises(smla.merge, po, pl[:, :2], match="part_lse must be")
    _raises(smla.merge, po, pl, out=_bf(3, 8, 512), match="out must be")
    _raises(smla.merge, po, pl, match="must be a GPU tensor")
    pool = torch.zeros((2, 256 * 656), dtype=torch.uint8)
    pages = torch.zeros(2, dtype=torch.int32)
    _raises(smla.split_pages_64, pool, pages, torch.zeros((7, 64 * 656), dtype=torch.uint8), match="4 pages per")
    _raises(smla.split_pages_64, pool, pages, torch.zeros((8, 64 * 600), dtype=torch.uint8), match="64 rows")
    _raises(smla.split_pages_64, pool, pages, torch.zeros((8, 64 * 656), dtype=torch.uint8), match="GPU tensor")
