// C ABI of the library: argument validation, workspace sizing and launches
// (host code only).
// Declarations and the contract of every entry point are in include/sparse_mla.h.
#include <stdarg.h>
#include <stdio.h>
#include <math.h>

#include "../../include/sparse_mla.h"
#include "../../include/sparse_mla_measure.h"
#include "common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxRows = 65535;  // query rows per call
constexpr int64_t kMaxBlocks = 0x7FFFFFFF;   // workgroups of one launch grid
// rows of the row-per-wavefront kernels (four rows per workgroup): at most
// 4 * kMaxBlocks, written so that no comparison can overflow
constexpr int64_t kMaxGridRows = 4 * kMaxBlocks;

}  // namespace

extern "C" {

const char* smla_last_error(void) { return g_err; }

int mla_kv_write(const void* kv_c, int64_t kv_c_row_stride, const void* k_pe,
                 int64_t k_pe_row_stride, int rope_dim, const int64_t* slot_mapping,
                 int64_t num_rows, void* kv_cache, int64_t num_slots, hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "mla_kv_write: rope_dim must be 0 or 64, got %d", rope_dim);
  if (num_rows < 0) return fail(SMLA_EINVAL, "mla_kv_write: num_rows < 0");
  if (num_slots < 1) return fail(SMLA_EINVAL, "mla_kv_write: num_slots must be >= 1");
  if (num_rows == 0) return SMLA_OK;
  if (num_rows > kMaxGridRows) return fail(SMLA_EUNSUPPORTED, "mla_kv_write: too many rows");
  if (kv_c == nullptr || slot_mapping == nullptr || kv_cache == nullptr)
    return fail(SMLA_EINVAL, "mla_kv_write: null pointer argument");
  if (rope_dim == 64 && k_pe == nullptr)
    return fail(SMLA_EINVAL, "mla_kv_write: k_pe is NULL with rope_dim 64");
  if (rope_dim == 0 && k_pe != nullptr)
    return fail(SMLA_EINVAL, "mla_kv_write: k_pe must be NULL with rope_dim 0");
  if (kv_c_row_stride < smla::kLatent || (kv_c_row_stride & 7))
    return fail(SMLA_EINVAL, "mla_kv_write: kv_c_row_stride must be >= 512 and a multiple of 8");
  if (rope_dim == 64 && (k_pe_row_stride < 64 || (k_pe_row_stride & 7)))
    return fail(SMLA_EINVAL, "mla_kv_write: k_pe_row_stride must be >= 64 and a multiple of 8");
  if (!aligned16(kv_c) || !aligned16(kv_cache) || (k_pe && !aligned16(k_pe)) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return fail(SMLA_EINVAL, "mla_kv_write: misaligned pointer");
  hipError_t e = smla::launch_kv_write(
      static_cast<const uint16_t*>(kv_c), kv_c_row_stride, static_cast<const uint16_t*>(k_pe),
      k_pe_row_stride, rope_dim, slot_mapping, num_rows, static_cast<uint8_t*>(kv_cache),
      num_slots, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "mla_kv_write: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int mla_kv_write_bf16(const void* kv_c, int64_t kv_c_row_stride, const void* k_pe,
                      int64_t k_pe_row_stride, int rope_dim, const int64_t* slot_mapping,
                      int64_t num_rows, void* kv_cache, int64_t num_slots, hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: rope_dim must be 0 or 64, got %d", rope_dim);
  if (num_rows < 0) return fail(SMLA_EINVAL, "mla_kv_write_bf16: num_rows < 0");
  if (num_slots < 1) return fail(SMLA_EINVAL, "mla_kv_write_bf16: num_slots must be >= 1");
  if (num_rows == 0) return SMLA_OK;
  if (num_rows > kMaxGridRows) return fail(SMLA_EUNSUPPORTED, "mla_kv_write_bf16: too many rows");
  if (kv_c == nullptr || slot_mapping == nullptr || kv_cache == nullptr)
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: null pointer argument");
  if (rope_dim == 64 && k_pe == nullptr)
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: k_pe is NULL with rope_dim 64");
  if (rope_dim == 0 && k_pe != nullptr)
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: k_pe must be NULL with rope_dim 0");
  if (kv_c_row_stride < smla::kLatent || (kv_c_row_stride & 7))
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: kv_c_row_stride must be >= 512 and a multiple of 8");
  if (rope_dim == 64 && (k_pe_row_stride < 64 || (k_pe_row_stride & 7)))
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: k_pe_row_stride must be >= 64 and a multiple of 8");
  if (!aligned16(kv_c) || !aligned16(kv_cache) || (k_pe && !aligned16(k_pe)) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return fail(SMLA_EINVAL, "mla_kv_write_bf16: misaligned pointer");
  hipError_t e = smla::launch_kv_write_bf16(
      static_cast<const uint16_t*>(kv_c), kv_c_row_stride, static_cast<const uint16_t*>(k_pe),
      k_pe_row_stride, rope_dim, slot_mapping, num_rows, static_cast<uint16_t*>(kv_cache),
      num_slots, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "mla_kv_write_bf16: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

size_t sparse_mla_attn_workspace_size(int T, int H, int topk_capacity, int rope_dim) {
  if (T < 1 || T > kMaxRows || H < 1 || H > SMLA_MAX_HEADS || topk_capacity < 1 ||
      (rope_dim != 0 && rope_dim != 64))
    return 0;
  const smla::AttnPlan plan = smla::plan_attn(T, H, topk_capacity, rope_dim);
  return plan.blocks > kMaxBlocks ? 0 : plan.workspace;
}

int sparse_mla_attn(const void* q, const void* kv_cache, int64_t num_slots,
                    const int32_t* topk_idx, int64_t idx_row_stride, int topk_capacity, int T,
                    int H, int rope_dim, float sm_scale, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "sparse_mla_attn: rope_dim must be 0 or 64, got %d", rope_dim);
  if (T < 1 || H < 1 || H > SMLA_MAX_HEADS)
    return fail(SMLA_EINVAL, "sparse_mla_attn: need T >= 1 and 1 <= H <= %d (T=%d, H=%d)",
                SMLA_MAX_HEADS, T, H);
  if (T > kMaxRows)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_attn: at most %d query rows per call", kMaxRows);
  if (topk_capacity < 1 || idx_row_stride < topk_capacity)
    return fail(SMLA_EINVAL, "sparse_mla_attn: need 1 <= topk_capacity <= idx_row_stride");
  if (num_slots < 1) return fail(SMLA_EINVAL, "sparse_mla_attn: num_slots must be >= 1");
  if (!isfinite(sm_scale)) return fail(SMLA_EINVAL, "sparse_mla_attn: sm_scale is not finite");
  if (q == nullptr || kv_cache == nullptr || topk_idx == nullptr || out == nullptr)
    return fail(SMLA_EINVAL, "sparse_mla_attn: null pointer argument");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(topk_idx) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SMLA_EINVAL, "sparse_mla_attn: misaligned pointer");
  const smla::AttnPlan plan = smla::plan_attn(T, H, topk_capacity, rope_dim);
  if (plan.blocks > kMaxBlocks)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_attn: %lld workgroups exceed one launch",
                (long long)plan.blocks);
  if (plan.workspace > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace)
      return fail(SMLA_EWORKSPACE, "sparse_mla_attn: workspace of %zu bytes needed, got %zu",
                  plan.workspace, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace)) return fail(SMLA_EINVAL, "sparse_mla_attn: misaligned workspace");
  }
  hipError_t e = smla::launch_attn(static_cast<const uint16_t*>(q),
                                   static_cast<const uint8_t*>(kv_cache), num_slots, topk_idx,
                                   idx_row_stride, topk_capacity, T, H, rope_dim, sm_scale,
                                   static_cast<uint16_t*>(out), lse, workspace, plan, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "sparse_mla_attn: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int sparse_mla_attn_noalloc(const void* q, const void* kv_cache, int64_t num_slots,
                            const int32_t* topk_idx, int64_t idx_row_stride, int topk_capacity, int T,
                            int H, int rope_dim, float sm_scale, void* out, float* lse,
                            hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: rope_dim must be 0 or 64, got %d", rope_dim);
  if (T < 1 || H < 1 || H > SMLA_MAX_HEADS)
    return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: need T >= 1 and 1 <= H <= %d (T=%d, H=%d)",
                SMLA_MAX_HEADS, T, H);
  if (T > kMaxRows)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_attn_noalloc: at most %d query rows per call", kMaxRows);
  if (topk_capacity < 1 || idx_row_stride < topk_capacity)
    return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: need 1 <= topk_capacity <= idx_row_stride");
  if (num_slots < 1) return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: num_slots must be >= 1");
  if (!isfinite(sm_scale)) return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: sm_scale is not finite");
  if (q == nullptr || kv_cache == nullptr || topk_idx == nullptr || out == nullptr)
    return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: null pointer argument");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(topk_idx) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SMLA_EINVAL, "sparse_mla_attn_noalloc: misaligned pointer");
  const smla::AttnPlan plan = smla::plan_attn(T, H, topk_capacity, rope_dim);
  if (plan.blocks > kMaxBlocks)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_attn_noalloc: %lld workgroups exceed one launch",
                (long long)plan.blocks);
  static_assert(smla::kNoallocScratchBytes == SMLA_NOALLOC_SCRATCH_BYTES, "scratch size");
  if (plan.workspace > smla::kNoallocScratchBytes)
    return fail(SMLA_EWORKSPACE,
                "sparse_mla_attn_noalloc: these sizes need %zu bytes of split partials, more than the "
                "%zu-byte scratch; call sparse_mla_attn with a workspace instead",
                plan.workspace, smla::kNoallocScratchBytes);
  void* scratch = nullptr;
  if (plan.workspace > 0) {
    const hipError_t se = smla::noalloc_scratch(stream, &scratch);
    if (se != hipSuccess)
      return fail(SMLA_ELAUNCH, "sparse_mla_attn_noalloc: no scratch on the stream's device: %s",
                  hipGetErrorString(se));
  }
  hipError_t e = smla::launch_attn(static_cast<const uint16_t*>(q),
                                   static_cast<const uint8_t*>(kv_cache), num_slots, topk_idx,
                                   idx_row_stride, topk_capacity, T, H, rope_dim, sm_scale,
                                   static_cast<uint16_t*>(out), lse, scratch, plan, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "sparse_mla_attn_noalloc: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int sparse_mla_attn_bf16(const void* q, const void* kv_cache, int64_t num_slots,
                         const int32_t* topk_idx, int64_t idx_row_stride, int topk_capacity, int T,
                         int H, int rope_dim, float sm_scale, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: rope_dim must be 0 or 64, got %d", rope_dim);
  if (T < 1 || H < 1 || H > SMLA_MAX_HEADS)
    return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: need T >= 1 and 1 <= H <= %d (T=%d, H=%d)",
                SMLA_MAX_HEADS, T, H);
  if (T > kMaxRows)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_attn_bf16: at most %d query rows per call", kMaxRows);
  if (topk_capacity < 1 || idx_row_stride < topk_capacity)
    return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: need 1 <= topk_capacity <= idx_row_stride");
  if (num_slots < 1) return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: num_slots must be >= 1");
  if (!isfinite(sm_scale)) return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: sm_scale is not finite");
  if (q == nullptr || kv_cache == nullptr || topk_idx == nullptr || out == nullptr)
    return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: null pointer argument");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(topk_idx) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: misaligned pointer");
  const smla::AttnPlan plan = smla::plan_attn(T, H, topk_capacity, rope_dim);
  if (plan.blocks > kMaxBlocks)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_attn_bf16: %lld workgroups exceed one launch",
                (long long)plan.blocks);
  if (plan.workspace > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace)
      return fail(SMLA_EWORKSPACE, "sparse_mla_attn_bf16: workspace of %zu bytes needed, got %zu",
                  plan.workspace, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace)) return fail(SMLA_EINVAL, "sparse_mla_attn_bf16: misaligned workspace");
  }
  hipError_t e = smla::launch_attn_bf16(static_cast<const uint16_t*>(q),
                                        static_cast<const uint16_t*>(kv_cache), num_slots, topk_idx,
                                        idx_row_stride, topk_capacity, T, H, rope_dim, sm_scale,
                                        static_cast<uint16_t*>(out), lse, workspace, plan, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "sparse_mla_attn_bf16: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int mla_gather_upconvert(const void* kv_cache, int64_t num_slots, int rope_dim,
                         const int64_t* slots, int64_t num_rows, void* dst, int64_t dst_row_stride,
                         hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "mla_gather_upconvert: rope_dim must be 0 or 64, got %d", rope_dim);
  if (num_rows < 0) return fail(SMLA_EINVAL, "mla_gather_upconvert: num_rows < 0");
  if (num_slots < 1) return fail(SMLA_EINVAL, "mla_gather_upconvert: num_slots must be >= 1");
  if (num_rows == 0) return SMLA_OK;
  if (num_rows > kMaxGridRows)
    return fail(SMLA_EUNSUPPORTED, "mla_gather_upconvert: too many rows");
  if (kv_cache == nullptr || slots == nullptr || dst == nullptr)
    return fail(SMLA_EINVAL, "mla_gather_upconvert: null pointer argument");
  if (dst_row_stride < 576 || (dst_row_stride & 7))
    return fail(SMLA_EINVAL, "mla_gather_upconvert: dst_row_stride must be >= 576 and a multiple of 8");
  if (!aligned16(kv_cache) || !aligned16(dst) || (reinterpret_cast<uintptr_t>(slots) & 7u))
    return fail(SMLA_EINVAL, "mla_gather_upconvert: misaligned pointer");
  hipError_t e = smla::launch_gather_upconvert(static_cast<const uint8_t*>(kv_cache), num_slots,
                                               rope_dim, slots, num_rows,
                                               static_cast<uint16_t*>(dst), dst_row_stride, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "mla_gather_upconvert: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int mla_split_pages_64(const void* src_pool, int64_t num_src_pages, int64_t src_page_stride,
                       const int32_t* pages, int64_t num_pages, void* dst, int64_t dst_page_stride,
                       int row_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if (row_bytes < 1)
    return fail(SMLA_EINVAL, "mla_split_pages_64: row_bytes must be positive, got %d", row_bytes);
  if (num_src_pages < 1 || num_pages < 0)
    return fail(SMLA_EINVAL, "mla_split_pages_64: need num_src_pages >= 1 and num_pages >= 0");
  if (num_pages == 0) return SMLA_OK;
  if (num_pages > kMaxBlocks / 4) return fail(SMLA_EUNSUPPORTED, "mla_split_pages_64: too many pages");
  if (src_pool == nullptr || pages == nullptr || dst == nullptr)
    return fail(SMLA_EINVAL, "mla_split_pages_64: null pointer argument");
  if (src_page_stride < 256 * (int64_t)row_bytes || (src_page_stride & 15))
    return fail(SMLA_EINVAL, "mla_split_pages_64: src_page_stride must be >= 256 * row_bytes and a multiple of 16");
  if (dst_page_stride < 64 * (int64_t)row_bytes || (dst_page_stride & 15))
    return fail(SMLA_EINVAL, "mla_split_pages_64: dst_page_stride must be >= 64 * row_bytes and a multiple of 16");
  if (!aligned16(src_pool) || !aligned16(dst) || (reinterpret_cast<uintptr_t>(pages) & 3u))
    return fail(SMLA_EINVAL, "mla_split_pages_64: misaligned pointer");
  hipError_t e = smla::launch_split_pages(static_cast<const uint8_t*>(src_pool), num_src_pages,
                                          src_page_stride, pages, num_pages,
                                          static_cast<uint8_t*>(dst), dst_page_stride, row_bytes, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "mla_split_pages_64: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int sparse_mla_merge(const void* part_out, const float* part_lse, int P, int T, int H, void* out,
                     float* lse, hipStream_t stream) {
  g_err[0] = '\0';
  if (P < 1 || T < 1 || H < 1 || H > SMLA_MAX_HEADS)
    return fail(SMLA_EINVAL, "sparse_mla_merge: need P >= 1, T >= 1 and 1 <= H <= %d (P=%d, T=%d, H=%d)",
                SMLA_MAX_HEADS, P, T, H);
  const int64_t rows = (int64_t)T * H;
  if (rows > kMaxGridRows)
    return fail(SMLA_EUNSUPPORTED, "sparse_mla_merge: too many (row, head) pairs");
  if (part_out == nullptr || part_lse == nullptr || out == nullptr)
    return fail(SMLA_EINVAL, "sparse_mla_merge: null pointer argument");
  if (!aligned16(part_out) || !aligned16(out) || (reinterpret_cast<uintptr_t>(part_lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SMLA_EINVAL, "sparse_mla_merge: misaligned pointer");
  hipError_t e = smla::launch_merge(static_cast<const uint16_t*>(part_out), part_lse, P, rows,
                                    static_cast<uint16_t*>(out), lse, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "sparse_mla_merge: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int smla_gather_rows_probe(const void* kv_cache, int64_t num_slots, int rope_dim, const int32_t* slots,
                           int64_t n, uint32_t* sink, hipStream_t stream) {
  g_err[0] = '\0';
  if (rope_dim != 0 && rope_dim != 64)
    return fail(SMLA_EINVAL, "smla_gather_rows_probe: rope_dim must be 0 or 64, got %d", rope_dim);
  if (n < 0 || num_slots < 1)
    return fail(SMLA_EINVAL, "smla_gather_rows_probe: need n >= 0 and num_slots >= 1");
  if (n > smla::gather_probe_max_rows())
    return fail(SMLA_EUNSUPPORTED, "smla_gather_rows_probe: at most %lld rows",
                (long long)smla::gather_probe_max_rows());
  if (n == 0) return SMLA_OK;
  if (kv_cache == nullptr || slots == nullptr || sink == nullptr)
    return fail(SMLA_EINVAL, "smla_gather_rows_probe: null pointer argument");
  if (!aligned16(kv_cache) || (reinterpret_cast<uintptr_t>(slots) & 3u) ||
      (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(SMLA_EINVAL, "smla_gather_rows_probe: misaligned pointer");
  hipError_t e = smla::launch_gather_probe(static_cast<const uint8_t*>(kv_cache), num_slots, rope_dim, slots,
                                           n, sink, stream);
  if (e != hipSuccess)
    return fail(SMLA_ELAUNCH, "smla_gather_rows_probe: launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

}  // extern "C"
