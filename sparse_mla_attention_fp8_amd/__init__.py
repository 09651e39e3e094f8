"""Python binding of libsparse_mla.so, the MI355X (gfx950) sparse-MLA library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/sparse_mla.h.  torch is used for
device memory (data_ptr) and the current stream; there is no fallback path,
and a missing or unloadable library raises.

    kv_write(kv_c, k_pe, slot_mapping, kv_cache)
    attn(q, kv_cache, topk_idx, sm_scale, rope_dim, topk_capacity=None,
         out=None, lse=None, workspace=None) -> (out, lse)
    merge(part_out, part_lse, out=None, lse=None) -> (out, lse)
    gather_upconvert(kv_cache, slots, rope_dim, out=None) -> out
    split_pages_64(src_pool, pages, dst, row_bytes=656)
    kv_write_bf16(kv_c, k_pe, slot_mapping, kv_cache_bf16)
    attn_bf16(q, kv_cache_bf16, topk_idx, sm_scale, ...) -> (out, lse)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_mla.so")

SMLA_OK, SMLA_EINVAL, SMLA_EWORKSPACE, SMLA_ELAUNCH, SMLA_EUNSUPPORTED = 0, -1, -2, -3, -4
ROW_BYTES = 656
LATENT = 512

# (name, restype, argtypes) of every exported entry point
_SIGS = {
    "mla_kv_write": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "sparse_mla_attn_workspace_size": (ctypes.c_size_t, [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "sparse_mla_attn": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_kv_write_bf16": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "sparse_mla_attn_bf16": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_gather_upconvert": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "mla_split_pages_64": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]),
    "sparse_mla_merge": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "smla_last_error": (ctypes.c_char_p, []),
}

_lib = None


class SparseMLAError(RuntimeError):
    def __init__(self, call: str, code: int, msg: str):
        super().__init__(f"{call} returned {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_mla_attention_fp8_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(call: str, rc: int) -> None:
    if rc != SMLA_OK:
        raise SparseMLAError(call, rc, lib().smla_last_error().decode())


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def kv_write(kv_c, k_pe, slot_mapping, kv_cache) -> None:
    """Quantise bf16 rows kv_c [N][>=512] (+ k_pe [N][>=64] or None) into
    kv_cache uint8 [num_slots][656] at slot_mapping int64 [N]; slot 0 dropped."""
    import torch
    assert kv_c.dtype == torch.bfloat16 and kv_c.dim() == 2 and kv_c.stride(1) == 1
    assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
    assert kv_cache.dtype == torch.uint8 and kv_cache.is_contiguous() and kv_cache.shape[-1] == ROW_BYTES
    rope_dim = 0
    pe_stride = 0
    if k_pe is not None:
        assert k_pe.dtype == torch.bfloat16 and k_pe.dim() == 2 and k_pe.stride(1) == 1
        rope_dim, pe_stride = 64, k_pe.stride(0)
    n = kv_c.shape[0]
    num_slots = kv_cache.numel() // ROW_BYTES
    rc = lib().mla_kv_write(kv_c.data_ptr(), kv_c.stride(0), _ptr(k_pe), pe_stride, rope_dim,
                            slot_mapping.data_ptr(), n, kv_cache.data_ptr(), num_slots,
                            _stream(kv_cache))
    _check("mla_kv_write", rc)


def workspace_size(T: int, H: int, topk_capacity: int, rope_dim: int) -> int:
    return int(lib().sparse_mla_attn_workspace_size(T, H, topk_capacity, rope_dim))


def attn(q, kv_cache, topk_idx, sm_scale: float, rope_dim: int, topk_capacity: int | None = None,
         out=None, lse=None, workspace=None, want_lse: bool = True):
    """Sparse MLA attention.  q bf16 [T][H][512+rope_dim]; kv_cache uint8
    [num_slots][656]; topk_idx int32 [T][>=W] (row stride may exceed W).
    Returns (out bf16 [T][H][512], lse float32 [T][H] or None)."""
    import torch
    assert q.dtype == torch.bfloat16 and q.dim() == 3 and q.is_contiguous()
    T, H, D = q.shape
    assert D == LATENT + rope_dim
    assert topk_idx.dtype == torch.int32 and topk_idx.dim() == 2 and topk_idx.stride(1) == 1
    assert kv_cache.dtype == torch.uint8 and kv_cache.is_contiguous()
    W = topk_idx.shape[1] if topk_capacity is None else int(topk_capacity)
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = workspace_size(T, H, W, rope_dim)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().sparse_mla_attn(q.data_ptr(), kv_cache.data_ptr(), kv_cache.numel() // ROW_BYTES,
                               topk_idx.data_ptr(), topk_idx.stride(0), W, T, H, rope_dim,
                               float(sm_scale), out.data_ptr(), _ptr(lse), _ptr(workspace),
                               ws_bytes, _stream(q))
    _check("sparse_mla_attn", rc)
    return out, lse


def merge(part_out, part_lse, out=None, lse=None, want_lse: bool = True):
    """Merge P partial results: part_out bf16 [P][T][H][512], part_lse float32
    [P][T][H].  Returns (out bf16 [T][H][512], lse float32 [T][H] or None)."""
    import torch
    assert part_out.dtype == torch.bfloat16 and part_out.dim() == 4 and part_out.is_contiguous()
    P, T, H, D = part_out.shape
    assert D == LATENT
    assert part_lse.dtype == torch.float32 and part_lse.is_contiguous() and tuple(part_lse.shape) == (P, T, H)
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=torch.bfloat16, device=part_out.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=part_out.device)
    rc = lib().sparse_mla_merge(part_out.data_ptr(), part_lse.data_ptr(), P, T, H, out.data_ptr(),
                                _ptr(lse), _stream(part_out))
    _check("sparse_mla_merge", rc)
    return out, lse


def gather_upconvert(kv_cache, slots, rope_dim: int, out=None):
    """Dequantise cache rows kv_cache uint8 [num_slots][656] at slots int64 [N]
    into bf16 [N][576] (out may be a wider row-strided view); invalid slots give
    zero rows, NoPE rows zeros in columns 512..575."""
    import torch
    assert kv_cache.dtype == torch.uint8 and kv_cache.is_contiguous() and kv_cache.shape[-1] == ROW_BYTES
    assert slots.dtype == torch.int64 and slots.dim() == 1 and slots.is_contiguous()
    n = slots.shape[0]
    if out is None:
        out = torch.empty((n, LATENT + 64), dtype=torch.bfloat16, device=kv_cache.device)
    assert out.dtype == torch.bfloat16 and out.dim() == 2 and out.stride(1) == 1 and out.shape[0] == n
    rc = lib().mla_gather_upconvert(kv_cache.data_ptr(), kv_cache.numel() // ROW_BYTES, rope_dim,
                                    slots.data_ptr(), n, out.data_ptr(), out.stride(0),
                                    _stream(kv_cache))
    _check("mla_gather_upconvert", rc)
    return out


def kv_write_bf16(kv_c, k_pe, slot_mapping, kv_cache) -> None:
    """Store bf16 rows kv_c [N][>=512] (+ k_pe [N][>=64] or None) into the BF16
    cache kv_cache bf16 [num_slots][512 + rope_dim] at slot_mapping int64 [N]."""
    import torch
    assert kv_c.dtype == torch.bfloat16 and kv_c.dim() == 2 and kv_c.stride(1) == 1
    assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
    rope_dim, pe_stride = 0, 0
    if k_pe is not None:
        assert k_pe.dtype == torch.bfloat16 and k_pe.dim() == 2 and k_pe.stride(1) == 1
        rope_dim, pe_stride = 64, k_pe.stride(0)
    assert kv_cache.dtype == torch.bfloat16 and kv_cache.is_contiguous()
    assert kv_cache.shape[-1] == LATENT + rope_dim
    rc = lib().mla_kv_write_bf16(kv_c.data_ptr(), kv_c.stride(0), _ptr(k_pe), pe_stride, rope_dim,
                                 slot_mapping.data_ptr(), kv_c.shape[0], kv_cache.data_ptr(),
                                 kv_cache.numel() // (LATENT + rope_dim), _stream(kv_cache))
    _check("mla_kv_write_bf16", rc)


def attn_bf16(q, kv_cache, topk_idx, sm_scale: float, topk_capacity: int | None = None,
              out=None, lse=None, workspace=None, want_lse: bool = True):
    """Sparse MLA attention over the BF16 cache kv_cache bf16 [num_slots][512 + rope_dim];
    q bf16 [T][H][512 + rope_dim] (rope_dim 0 or 64, read from q's width);
    topk_idx int32 [T][>=W]."""
    import torch
    assert q.dtype == torch.bfloat16 and q.dim() == 3 and q.is_contiguous()
    rope_dim = q.shape[2] - LATENT
    assert rope_dim in (0, 64)
    assert kv_cache.dtype == torch.bfloat16 and kv_cache.is_contiguous() and kv_cache.shape[-1] == q.shape[2]
    assert topk_idx.dtype == torch.int32 and topk_idx.dim() == 2 and topk_idx.stride(1) == 1
    T, H, _ = q.shape
    W = topk_idx.shape[1] if topk_capacity is None else int(topk_capacity)
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = workspace_size(T, H, W, rope_dim)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().sparse_mla_attn_bf16(q.data_ptr(), kv_cache.data_ptr(), kv_cache.numel() // q.shape[2],
                                    topk_idx.data_ptr(), topk_idx.stride(0), W, T, H, rope_dim,
                                    float(sm_scale), out.data_ptr(), _ptr(lse), _ptr(workspace),
                                    ws_bytes, _stream(q))
    _check("sparse_mla_attn_bf16", rc)
    return out, lse


def split_pages_64(src_pool, pages, dst, row_bytes: int = ROW_BYTES) -> None:
    """Copy the listed 256-token pages of src_pool (uint8 [num_src_pages][>=256*row_bytes])
    into 64-token pages of dst (uint8 [>=4*num_src_pages][>=64*row_bytes], zeroed
    by the caller at allocation); pages int32 [n]."""
    import torch
    assert src_pool.dtype == torch.uint8 and src_pool.dim() == 2 and src_pool.stride(1) == 1
    assert dst.dtype == torch.uint8 and dst.dim() == 2 and dst.stride(1) == 1
    assert pages.dtype == torch.int32 and pages.dim() == 1 and pages.is_contiguous()
    assert dst.shape[0] >= 4 * src_pool.shape[0]
    rc = lib().mla_split_pages_64(src_pool.data_ptr(), src_pool.shape[0], src_pool.stride(0),
                                  pages.data_ptr(), pages.shape[0], dst.data_ptr(), dst.stride(0),
                                  int(row_bytes), _stream(src_pool))
    _check("mla_split_pages_64", rc)
