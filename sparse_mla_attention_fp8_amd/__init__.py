"""Python binding of libsparse_mla.so, the MI355X (gfx950) sparse-MLA library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/sparse_mla.h.  torch is used for
device memory (data_ptr) and the current stream; there is no fallback path,
and a missing or unloadable library raises.

    kv_write(kv_c, k_pe, slot_mapping, kv_cache)
    attn(q, kv_cache, topk_idx, sm_scale, rope_dim, topk_capacity=None,
         out=None, lse=None, workspace=None) -> (out, lse)
    attn_noalloc(q, kv_cache, topk_idx, sm_scale, rope_dim, topk_capacity=None,
                 out, lse=None) -> (out, lse)
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
NOALLOC_SCRATCH_BYTES = 16 << 20
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
    "sparse_mla_attn_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
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
    "smla_gather_rows_probe": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p]),
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


def _need(call: str, cond: bool, msg: str) -> None:
    """Argument check of the binding; raises before anything is launched."""
    if not cond:
        raise ValueError(f"{call}: {msg}")


def _same_device(call: str, ref_name: str, ref, **others) -> None:
    """Every tensor must live on the reference tensor's GPU: a host tensor's
    data_ptr() handed to a kernel would be dereferenced as a device address."""
    _need(call, ref.is_cuda, f"{ref_name} must be a GPU tensor (it is on {ref.device})")
    for name, t in others.items():
        if t is not None:
            _need(call, t.device == ref.device, f"{name} is on {t.device}, {ref_name} on {ref.device}")


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _check_rows_bf16(call: str, name: str, t, min_width: int) -> None:
    import torch
    _need(call, t.dtype == torch.bfloat16 and t.dim() == 2 and t.stride(1) == 1,
          f"{name} must be a 2-D bf16 tensor with unit column stride")
    _need(call, t.shape[1] >= min_width, f"{name} rows must hold >= {min_width} values (got {t.shape[1]})")


def _check_out_lse(call: str, out, lse, T: int, H: int) -> None:
    import torch
    if out is not None:
        _need(call, out.dtype == torch.bfloat16 and tuple(out.shape) == (T, H, LATENT) and out.is_contiguous(),
              f"out must be a contiguous bf16 [{T}][{H}][{LATENT}] tensor")
    if lse is not None:
        _need(call, lse.dtype == torch.float32 and tuple(lse.shape) == (T, H) and lse.is_contiguous(),
              f"lse must be a contiguous float32 [{T}][{H}] tensor")


def _check_topk(call: str, topk_idx, T: int, topk_capacity) -> int:
    import torch
    _need(call, topk_idx.dtype == torch.int32 and topk_idx.dim() == 2 and topk_idx.stride(1) == 1,
          "topk_idx must be a 2-D int32 tensor with unit column stride")
    _need(call, topk_idx.shape[0] == T, f"topk_idx has {topk_idx.shape[0]} rows for {T} query rows")
    W = topk_idx.shape[1] if topk_capacity is None else int(topk_capacity)
    _need(call, 1 <= W <= topk_idx.shape[1],
          f"topk_capacity {W} must be in [1, {topk_idx.shape[1]}] (the buffer's width)")
    return W


def _check_workspace(call: str, workspace) -> None:
    if workspace is not None:
        _need(call, workspace.is_contiguous(), "workspace must be contiguous")


def kv_write(kv_c, k_pe, slot_mapping, kv_cache) -> None:
    """Quantise bf16 rows kv_c [N][>=512] (+ k_pe [N][>=64] or None) into
    kv_cache uint8 [num_slots][656] at slot_mapping int64 [N]; slot 0 dropped."""
    import torch
    call = "kv_write"
    _check_rows_bf16(call, "kv_c", kv_c, LATENT)
    n = kv_c.shape[0]
    _need(call, slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
          "slot_mapping must be a contiguous 1-D int64 tensor")
    _need(call, slot_mapping.shape[0] == n, f"slot_mapping has {slot_mapping.shape[0]} entries for {n} rows")
    _need(call, kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == ROW_BYTES, f"kv_cache must be a contiguous uint8 [num_slots][{ROW_BYTES}] tensor")
    rope_dim, pe_stride = 0, 0
    if k_pe is not None:
        _check_rows_bf16(call, "k_pe", k_pe, 64)
        _need(call, k_pe.shape[0] == n, f"k_pe has {k_pe.shape[0]} rows for {n} rows of kv_c")
        rope_dim, pe_stride = 64, k_pe.stride(0)
    _same_device(call, "kv_cache", kv_cache, kv_c=kv_c, k_pe=k_pe, slot_mapping=slot_mapping)
    rc = lib().mla_kv_write(kv_c.data_ptr(), kv_c.stride(0), _ptr(k_pe), pe_stride, rope_dim,
                            slot_mapping.data_ptr(), n, kv_cache.data_ptr(), kv_cache.shape[0],
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
    call = "attn"
    _need(call, rope_dim in (0, 64), f"rope_dim must be 0 or 64, got {rope_dim}")
    _need(call, q.dtype == torch.bfloat16 and q.dim() == 3 and q.is_contiguous(),
          "q must be a contiguous 3-D bf16 tensor")
    T, H, D = q.shape
    _need(call, D == LATENT + rope_dim, f"q rows are {D} wide, expected {LATENT + rope_dim} for rope_dim {rope_dim}")
    W = _check_topk(call, topk_idx, T, topk_capacity)
    _need(call, kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == ROW_BYTES, f"kv_cache must be a contiguous uint8 [num_slots][{ROW_BYTES}] tensor")
    _check_out_lse(call, out, lse, T, H)
    _check_workspace(call, workspace)
    _same_device(call, "q", q, kv_cache=kv_cache, topk_idx=topk_idx, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = workspace_size(T, H, W, rope_dim)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if need and ws_bytes < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = need
    rc = lib().sparse_mla_attn(q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
                               topk_idx.data_ptr(), topk_idx.stride(0), W, T, H, rope_dim,
                               float(sm_scale), out.data_ptr(), _ptr(lse), _ptr(workspace),
                               ws_bytes, _stream(q))
    _check("sparse_mla_attn", rc)
    return out, lse


def attn_noalloc(q, kv_cache, topk_idx, sm_scale: float, rope_dim: int, out, lse=None,
                 topk_capacity: int | None = None):
    """sparse_mla_attn_noalloc: attn() without a workspace; the library's
    per-GPU scratch holds the split partials, and the caller passes out (and
    lse) so that the call allocates nothing.  Calls that overlap on one GPU
    race on that scratch."""
    import torch
    call = "attn_noalloc"
    _need(call, rope_dim in (0, 64), f"rope_dim must be 0 or 64, got {rope_dim}")
    _need(call, q.dtype == torch.bfloat16 and q.dim() == 3 and q.is_contiguous(),
          "q must be a contiguous 3-D bf16 tensor")
    T, H, D = q.shape
    _need(call, D == LATENT + rope_dim, f"q rows are {D} wide, expected {LATENT + rope_dim} for rope_dim {rope_dim}")
    W = _check_topk(call, topk_idx, T, topk_capacity)
    _need(call, kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == ROW_BYTES, f"kv_cache must be a contiguous uint8 [num_slots][{ROW_BYTES}] tensor")
    _need(call, out is not None, "out must be given (the call allocates nothing)")
    _check_out_lse(call, out, lse, T, H)
    _same_device(call, "q", q, kv_cache=kv_cache, topk_idx=topk_idx, out=out, lse=lse)
    rc = lib().sparse_mla_attn_noalloc(q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
                                       topk_idx.data_ptr(), topk_idx.stride(0), W, T, H, rope_dim,
                                       float(sm_scale), out.data_ptr(), _ptr(lse), _stream(q))
    _check("sparse_mla_attn_noalloc", rc)
    return out, lse


def merge(part_out, part_lse, out=None, lse=None, want_lse: bool = True):
    """Merge P partial results: part_out bf16 [P][T][H][512], part_lse float32
    [P][T][H].  Returns (out bf16 [T][H][512], lse float32 [T][H] or None)."""
    import torch
    call = "merge"
    _need(call, part_out.dtype == torch.bfloat16 and part_out.dim() == 4 and part_out.is_contiguous(),
          "part_out must be a contiguous 4-D bf16 tensor")
    P, T, H, D = part_out.shape
    _need(call, D == LATENT, f"part_out rows are {D} wide, expected {LATENT}")
    _need(call, part_lse.dtype == torch.float32 and part_lse.is_contiguous() and tuple(part_lse.shape) == (P, T, H),
          f"part_lse must be a contiguous float32 [{P}][{T}][{H}] tensor")
    _check_out_lse(call, out, lse, T, H)
    _same_device(call, "part_out", part_out, part_lse=part_lse, out=out, lse=lse)
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
    call = "gather_upconvert"
    _need(call, rope_dim in (0, 64), f"rope_dim must be 0 or 64, got {rope_dim}")
    _need(call, kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == ROW_BYTES, f"kv_cache must be a contiguous uint8 [num_slots][{ROW_BYTES}] tensor")
    _need(call, slots.dtype == torch.int64 and slots.dim() == 1 and slots.is_contiguous(),
          "slots must be a contiguous 1-D int64 tensor")
    n = slots.shape[0]
    if out is not None:
        _check_rows_bf16(call, "out", out, LATENT + 64)
        _need(call, out.shape[0] == n, f"out has {out.shape[0]} rows for {n} slots")
    _same_device(call, "kv_cache", kv_cache, slots=slots, out=out)
    if out is None:
        out = torch.empty((n, LATENT + 64), dtype=torch.bfloat16, device=kv_cache.device)
    rc = lib().mla_gather_upconvert(kv_cache.data_ptr(), kv_cache.shape[0], rope_dim,
                                    slots.data_ptr(), n, out.data_ptr(), out.stride(0),
                                    _stream(kv_cache))
    _check("mla_gather_upconvert", rc)
    return out


def kv_write_bf16(kv_c, k_pe, slot_mapping, kv_cache) -> None:
    """Store bf16 rows kv_c [N][>=512] (+ k_pe [N][>=64] or None) into the BF16
    cache kv_cache bf16 [num_slots][512 + rope_dim] at slot_mapping int64 [N]."""
    import torch
    call = "kv_write_bf16"
    _check_rows_bf16(call, "kv_c", kv_c, LATENT)
    n = kv_c.shape[0]
    _need(call, slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1 and slot_mapping.is_contiguous(),
          "slot_mapping must be a contiguous 1-D int64 tensor")
    _need(call, slot_mapping.shape[0] == n, f"slot_mapping has {slot_mapping.shape[0]} entries for {n} rows")
    rope_dim, pe_stride = 0, 0
    if k_pe is not None:
        _check_rows_bf16(call, "k_pe", k_pe, 64)
        _need(call, k_pe.shape[0] == n, f"k_pe has {k_pe.shape[0]} rows for {n} rows of kv_c")
        rope_dim, pe_stride = 64, k_pe.stride(0)
    _need(call, kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == LATENT + rope_dim,
          f"kv_cache must be a contiguous bf16 [num_slots][{LATENT + rope_dim}] tensor")
    _same_device(call, "kv_cache", kv_cache, kv_c=kv_c, k_pe=k_pe, slot_mapping=slot_mapping)
    rc = lib().mla_kv_write_bf16(kv_c.data_ptr(), kv_c.stride(0), _ptr(k_pe), pe_stride, rope_dim,
                                 slot_mapping.data_ptr(), n, kv_cache.data_ptr(),
                                 kv_cache.shape[0], _stream(kv_cache))
    _check("mla_kv_write_bf16", rc)


def attn_bf16(q, kv_cache, topk_idx, sm_scale: float, topk_capacity: int | None = None,
              out=None, lse=None, workspace=None, want_lse: bool = True):
    """Sparse MLA attention over the BF16 cache kv_cache bf16 [num_slots][512 + rope_dim];
    q bf16 [T][H][512 + rope_dim] (rope_dim 0 or 64, read from q's width);
    topk_idx int32 [T][>=W]."""
    import torch
    call = "attn_bf16"
    _need(call, q.dtype == torch.bfloat16 and q.dim() == 3 and q.is_contiguous(),
          "q must be a contiguous 3-D bf16 tensor")
    T, H, D = q.shape
    rope_dim = D - LATENT
    _need(call, rope_dim in (0, 64), f"q rows must be {LATENT} or {LATENT + 64} wide, got {D}")
    _need(call, kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == D, f"kv_cache must be a contiguous bf16 [num_slots][{D}] tensor")
    W = _check_topk(call, topk_idx, T, topk_capacity)
    _check_out_lse(call, out, lse, T, H)
    _check_workspace(call, workspace)
    _same_device(call, "q", q, kv_cache=kv_cache, topk_idx=topk_idx, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = workspace_size(T, H, W, rope_dim)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if need and ws_bytes < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = need
    rc = lib().sparse_mla_attn_bf16(q.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
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
    call = "split_pages_64"
    _need(call, src_pool.dtype == torch.uint8 and src_pool.dim() == 2 and src_pool.stride(1) == 1,
          "src_pool must be a 2-D uint8 tensor with unit column stride")
    _need(call, dst.dtype == torch.uint8 and dst.dim() == 2 and dst.stride(1) == 1,
          "dst must be a 2-D uint8 tensor with unit column stride")
    _need(call, pages.dtype == torch.int32 and pages.dim() == 1 and pages.is_contiguous(),
          "pages must be a contiguous 1-D int32 tensor")
    _need(call, src_pool.shape[1] >= 256 * row_bytes, f"src_pool pages must hold 256 rows of {row_bytes} bytes")
    _need(call, dst.shape[1] >= 64 * row_bytes, f"dst pages must hold 64 rows of {row_bytes} bytes")
    _need(call, dst.shape[0] >= 4 * src_pool.shape[0], "dst must hold 4 pages per source page")
    _same_device(call, "src_pool", src_pool, pages=pages, dst=dst)
    rc = lib().mla_split_pages_64(src_pool.data_ptr(), src_pool.shape[0], src_pool.stride(0),
                                  pages.data_ptr(), pages.shape[0], dst.data_ptr(), dst.stride(0),
                                  int(row_bytes), _stream(src_pool))
    _check("mla_split_pages_64", rc)


def gather_rows_probe(kv_cache, slots, rope_dim: int, sink=None):
    """smla_gather_rows_probe: read the bytes of the listed rows (int32 slots
    [n]) that an attention call gathers, with no arithmetic; for measuring the
    gather ceiling of a list of rows.  Returns the uint32 sink tensor."""
    import torch
    call = "gather_rows_probe"
    _need(call, rope_dim in (0, 64), f"rope_dim must be 0 or 64, got {rope_dim}")
    _need(call, kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.is_contiguous()
          and kv_cache.shape[1] == ROW_BYTES, f"kv_cache must be a contiguous uint8 [num_slots][{ROW_BYTES}] tensor")
    _need(call, slots.dtype == torch.int32 and slots.dim() == 1 and slots.is_contiguous(),
          "slots must be a contiguous 1-D int32 tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=kv_cache.device)
    _need(call, sink.numel() >= 1 and sink.element_size() == 4, "sink must hold one 32-bit word")
    _same_device(call, "kv_cache", kv_cache, slots=slots, sink=sink)
    rc = lib().smla_gather_rows_probe(kv_cache.data_ptr(), kv_cache.shape[0], rope_dim, slots.data_ptr(),
                                      slots.shape[0], sink.data_ptr(), _stream(kv_cache))
    _check("smla_gather_rows_probe", rc)
    return sink
