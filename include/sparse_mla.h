/*
 * sparse_mla.h - C ABI of the MI355X (gfx950) sparse-MLA library.
 *
 * Two calls make up the hot path of DeepSeek/GLM-style sparse MLA decoding
 * over a paged FP8 KV cache:
 *
 *   mla_kv_write     packs bf16 latent rows (+ optional RoPE) into 656-byte
 *                    fp8_ds_mla cache rows, dropping writes aimed at the
 *                    reserved padding slot 0;
 *   sparse_mla_attn  attends every query row over its top-k list of cache
 *                    slots, where a negative entry is padding.
 *
 * the same two over a BF16 KV cache (rows of bf16 values, no quantisation):
 *
 *   mla_kv_write_bf16, sparse_mla_attn_bf16;
 *
 * the attention call without a caller workspace, for callers that cannot
 * allocate:
 *
 *   sparse_mla_attn_noalloc;
 *
 * and three more around them:
 *
 *   mla_gather_upconvert  dequantises listed cache rows into a bf16 workspace
 *                         of 576-wide rows (the chunked-context reader's form);
 *   sparse_mla_merge      merges partial (out, lse) pairs of sparse_mla_attn
 *                         calls over disjoint shares of the top-k entries
 *                         (context-parallel decoding) by their log-sum-exp;
 *   mla_split_pages_64    re-pages the touched 256-token pages of a pool into
 *                         a zero-initialised scratch of 64-token pages.
 *
 * Common rules
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library allocates nothing and keeps no device state between calls,
 *     except the per-GPU scratch array of sparse_mla_attn_noalloc.
 *   - Calls are asynchronous on `stream` (0 = the null stream) and do not
 *     synchronise.  They are reentrant; concurrent calls on different streams
 *     must not write the same memory.
 *   - Argument errors are detected on the host before any launch and return a
 *     negative code; nothing is launched then.  smla_last_error() returns a
 *     thread-local text for the last failing call on the calling thread.
 *   - Device-side values (slots, indices) are not validated beyond the rules
 *     stated per call; out-of-range ones are treated as "drop" / "padding".
 *   - Offsets into the cache are 64-bit: slot * 656 does not wrap.
 *   - Results are bitwise reproducible for the same inputs and sizes
 *     (no floating-point atomics, fixed reduction order).
 *
 * Cache layout (vLLM PR 55277, "Support NoPE sparse MLA (GLM-5.3-Flash) on
 * the FlashInfer SM120 backend", Purpose (1)): the cache is uint8
 * [num_slots][656], slot = page * 64 + offset for 64-token pages
 * (sglang PR 39288, Root cause (2)).  Row bytes:
 *   [0, 512)    e4m3 codes (OCP "fn" encoding, NaN = 0x7F / 0xFF) of the
 *               512-wide latent, four tiles of 128 values;
 *   [512, 528)  the four tile scales, float32 little-endian, tile order;
 *   [528, 656)  64 bf16 RoPE values, or zeros for NoPE rows (rope_dim 0).
 */
#ifndef SPARSE_MLA_H
#define SPARSE_MLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

/* The library exports its entry points and nothing else. */
#ifndef SMLA_API
#define SMLA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_OK            0
#define SMLA_EINVAL       -1  /* bad argument (null pointer, size, alignment, rope_dim) */
#define SMLA_EWORKSPACE   -2  /* workspace smaller than sparse_mla_attn_workspace_size() */
#define SMLA_ELAUNCH      -3  /* the HIP runtime reported an error at launch */
#define SMLA_EUNSUPPORTED -4  /* a size the library does not handle */

#define SMLA_ROW_BYTES   656
#define SMLA_LATENT      512
#define SMLA_MAX_HEADS   128

/*
 * mla_kv_write - quantise and store MLA KV rows.
 *
 * Follows sglang PR 47013 ("zero-RoPE MLA KV writer skips reserved slot 0"),
 * Summary and Modifications, and vLLM PR 55277, Purpose (1):
 *   for each row i with 1 <= slot_mapping[i] < num_slots:
 *     per 128-value tile t of the latent: amax_t = max |x|,
 *       scale_t = fp32(amax_t / 448)  (IEEE float32 division);
 *     code = e4m3(fp32(x / scale_t)), rounded to nearest even, saturating at
 *       +-448; a tile with amax_t == 0 stores scale 0 and all-zero codes;
 *     bytes [528,656) = the 64 RoPE values (rope_dim 64) or zeros (rope_dim 0).
 *   Rows whose slot is 0 (the reserved padding slot), negative or
 *   >= num_slots are dropped and their inputs are never read, so padding
 *   rows may hold NaN.  No other cache byte is written.  Duplicate slots in
 *   one call leave that slot holding one of the rows (unspecified which).
 *   NaN inputs in kept rows are not sanitised.
 *
 * kv_c            bf16 [num_rows][>= 512], row stride kv_c_row_stride elements
 *                 (multiple of 8), base 16-byte aligned.
 * k_pe            bf16 [num_rows][>= 64] with stride k_pe_row_stride (multiple
 *                 of 8, base 16-byte aligned) when rope_dim == 64; must be NULL
 *                 when rope_dim == 0.
 * rope_dim        64 or 0; anything else is SMLA_EINVAL.
 * slot_mapping    int64 [num_rows].
 * num_rows        >= 0 (0 launches nothing).
 * kv_cache        uint8 [num_slots][656], 16-byte aligned; num_slots >= 1.
 */
SMLA_API int mla_kv_write(const void* kv_c, int64_t kv_c_row_stride,
                 const void* k_pe, int64_t k_pe_row_stride,
                 int rope_dim,
                 const int64_t* slot_mapping, int64_t num_rows,
                 void* kv_cache, int64_t num_slots,
                 hipStream_t stream);

/*
 * sparse_mla_attn_workspace_size - bytes of device workspace that
 * sparse_mla_attn needs for these sizes (0 when none is needed).  Pure host
 * function; returns 0 for invalid sizes as well (sparse_mla_attn reports them).
 */
SMLA_API size_t sparse_mla_attn_workspace_size(int T, int H, int topk_capacity, int rope_dim);

/*
 * sparse_mla_attn - sparse MLA attention over the fp8_ds_mla cache.
 *
 * Follows sglang PR 47013, Motivation; sglang PR 39288 ("zero-initialise the
 * 64-token page-split scratch so masked candidates never gather NaN from
 * slot 0"), Root cause (1); and vLLM PR 55277, Purpose (1) and (2):
 *   for query row t and head h, over the valid entries j of topk_idx[t][0..W)
 *   (valid: 0 <= idx < num_slots; any other value is padding, anywhere in the
 *   row; duplicates count once per entry):
 *     K_j[e]     = e4m3(code[e]) * scale[e / 128]    (e < 512)
 *     K_j[512+r] = RoPE value r                      (rope_dim 64 only)
 *     s_j = sm_scale * sum_d q[t][h][d] * K_j[d], d < 512 + rope_dim
 *     out[t][h] = sum_j softmax(s)_j * K_j[0..512)
 *     lse[t][h] = ln sum_j exp(s_j)
 *   A row with no valid entry gives out = 0 and lse = -inf.  Padding entries
 *   are never loaded and contribute exactly zero, whatever bytes slot 0 or any
 *   unreferenced slot holds (NaN codes included).  NoPE (rope_dim 0) scores
 *   use 512 dims and never read row bytes [528, 656).
 *
 * q               bf16 [T][H][512 + rope_dim], contiguous, 16-byte aligned.
 * kv_cache        uint8 [num_slots][656], 16-byte aligned; num_slots >= 1.
 * topk_idx        int32 [T][idx_row_stride]; only the first topk_capacity
 *                 entries of a row are read.  topk_capacity is the buffer's
 *                 width (e.g. 2176 = index_topk 2048 + a 128-wide tail); the
 *                 -1 padding bounds the active length.  1 <= topk_capacity <=
 *                 idx_row_stride.
 * T, H            1 <= T, 1 <= H <= 128.
 * rope_dim        64 or 0.
 * sm_scale        softmax scale (e.g. 1/sqrt(576)), finite.
 * out             bf16 [T][H][512], 16-byte aligned.
 * lse             float32 [T][H] natural-log LSE, or NULL.
 * workspace       device memory of >= sparse_mla_attn_workspace_size(T, H,
 *                 topk_capacity, rope_dim) bytes (16-byte aligned), or NULL
 *                 when that size is 0.  Its contents on entry do not matter
 *                 (split partials, and with two or three splits per row the
 *                 words that find the split finishing last, which each call
 *                 leaves zero); two calls that share it must not overlap.
 */
SMLA_API int sparse_mla_attn(const void* q,
                    const void* kv_cache, int64_t num_slots,
                    const int32_t* topk_idx, int64_t idx_row_stride, int topk_capacity,
                    int T, int H, int rope_dim, float sm_scale,
                    void* out, float* lse,
                    void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * sparse_mla_attn_noalloc - sparse_mla_attn without a caller workspace.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation, kernels and arguments as sparse_mla_attn, minus the workspace:
 * the split partials go to a scratch array of SMLA_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc, no hipFree).  Its first use on a device
 * looks the array's address up once (hipGetSymbolAddress, briefly making the
 * stream's device current if it is not).
 *
 * Limit: sizes whose split partials would exceed the scratch, i.e.
 * sparse_mla_attn_workspace_size(T, H, topk_capacity, rope_dim) >
 * SMLA_NOALLOC_SCRATCH_BYTES, return SMLA_EWORKSPACE before any launch (every
 * size with topk_capacity <= 2304 fits: it needs at most 8.03 MiB).
 * All calls on one GPU share its scratch: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must not be issued.
 * Nothing in the scratch needs to start at zero (with two or three splits per
 * row it also holds the words that find the split finishing last, which each
 * call leaves zero).
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (16u << 20)
SMLA_API int sparse_mla_attn_noalloc(const void* q,
                            const void* kv_cache, int64_t num_slots,
                            const int32_t* topk_idx, int64_t idx_row_stride, int topk_capacity,
                            int T, int H, int rope_dim, float sm_scale,
                            void* out, float* lse,
                            hipStream_t stream);

/*
 * mla_kv_write_bf16 - store MLA KV rows into a BF16 KV cache.
 *
 * The BF16 cache of sglang PR 47013, Speed Tests (its timed writer stores rows
 * of 512 bf16 values; the end-to-end runs there use a BF16 KV cache): row
 * slot of kv_cache (bf16 [num_slots][512 + rope_dim]) receives kv_c[i][0..512)
 * and, with rope_dim 64, k_pe[i][0..64), unchanged.  The slot rule of
 * mla_kv_write applies: slot 0, negative slots and slots >= num_slots are
 * dropped and their inputs never read.  Arguments as for mla_kv_write, except
 * kv_cache: bf16 [num_slots][512 + rope_dim], 16-byte aligned.
 */
SMLA_API int mla_kv_write_bf16(const void* kv_c, int64_t kv_c_row_stride,
                      const void* k_pe, int64_t k_pe_row_stride,
                      int rope_dim,
                      const int64_t* slot_mapping, int64_t num_rows,
                      void* kv_cache, int64_t num_slots,
                      hipStream_t stream);

/*
 * sparse_mla_attn_bf16 - sparse MLA attention over a BF16 KV cache.
 *
 * The computation of sparse_mla_attn with K_j[e] = the bf16 value stored at
 * kv_cache[j][e] (no dequantisation): kv_cache is bf16 [num_slots][512 +
 * rope_dim] as mla_kv_write_bf16 writes it, 16-byte aligned, and q is bf16
 * [T][H][512 + rope_dim]; scores run over all 512 + rope_dim dimensions, the
 * output over the 512 latent ones.  All other arguments, the padding rules,
 * the workspace (same size as sparse_mla_attn_workspace_size) and the error
 * behaviour are those of sparse_mla_attn.
 */
SMLA_API int sparse_mla_attn_bf16(const void* q,
                         const void* kv_cache, int64_t num_slots,
                         const int32_t* topk_idx, int64_t idx_row_stride, int topk_capacity,
                         int T, int H, int rope_dim, float sm_scale,
                         void* out, float* lse,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * mla_gather_upconvert - dequantise listed cache rows into bf16 rows.
 *
 * Follows vLLM PR 55277, Purpose (1), and the review of that PR on the cache
 * gather for the chunked-context path: with rope_dim 0 the reader must see
 * exact zeros in columns 512..575, never stale cache bytes.  For each i:
 *   if 0 <= slots[i] < num_slots, with row = kv_cache[slots[i]]:
 *     dst[i][e]       = bf16(fp32(e4m3(code[e]) * scale[e / 128]))  (e < 512)
 *     dst[i][512 + r] = RoPE value r (rope_dim 64), or +0 (rope_dim 0; row
 *                       bytes [528, 656) are then not read)
 *   otherwise (negative or >= num_slots) dst[i][0..576) = +0.
 *   The dequantised value is rounded to float32, then to bf16, both to
 *   nearest even; NaN codes give the bf16 NaN 0x7FC0.  Slot 0 is read like
 *   any other slot.
 *
 * kv_cache        uint8 [num_slots][656], 16-byte aligned; num_slots >= 1.
 * rope_dim        64 or 0 (the layout of the cache rows).
 * slots           int64 [num_rows], 8-byte aligned.
 * num_rows        >= 0 (0 launches nothing).
 * dst             bf16 [num_rows][dst_row_stride], 16-byte aligned; columns
 *                 576 .. dst_row_stride-1 are not written.
 * dst_row_stride  elements, >= 576 and a multiple of 8.
 */
SMLA_API int mla_gather_upconvert(const void* kv_cache, int64_t num_slots, int rope_dim,
                         const int64_t* slots, int64_t num_rows,
                         void* dst, int64_t dst_row_stride, hipStream_t stream);

/*
 * mla_split_pages_64 - re-page 256-token pages into a 64-token scratch.
 *
 * Follows sglang PR 39288, Root cause (2) and Modifications: a pool of
 * 256-token pages is re-paged for a reader of 64-token pages by copying each
 * source page a step references into four 64-token pages of a persistent
 * scratch.  The scratch must be zero-filled by the caller when it is
 * allocated (the pages' fix), so that its slot 0 is finite whether or not
 * source page 0 is ever copied; this call copies and never clears.  For
 * every listed page p with 0 <= p < num_src_pages (other entries are
 * ignored; duplicates copy the same bytes twice) and k = 0..3:
 *   dst + (4p + k) * dst_page_stride, 64 * row_bytes bytes
 *     = src_pool + p * src_page_stride + k * 64 * row_bytes
 * No other byte of dst is written (untouched pages and the padding past
 * 64 * row_bytes in each dst page keep their contents).
 *
 * src_pool        uint8, num_src_pages pages of src_page_stride bytes
 *                 (>= 256 * row_bytes, a multiple of 16), 16-byte aligned.
 * pages           int32 [num_pages], the touched source pages.
 * dst             uint8, >= 4 * num_src_pages pages of dst_page_stride bytes
 *                 (>= 64 * row_bytes, a multiple of 16), 16-byte aligned.
 * row_bytes       bytes per token row, >= 1 (656 for fp8_ds_mla; any size,
 *                 e.g. 585 for the 37,440-byte 64-token page, since 64 rows
 *                 always span a multiple of 16 bytes).
 */
SMLA_API int mla_split_pages_64(const void* src_pool, int64_t num_src_pages, int64_t src_page_stride,
                       const int32_t* pages, int64_t num_pages,
                       void* dst, int64_t dst_page_stride, int row_bytes,
                       hipStream_t stream);

/*
 * sparse_mla_merge - combine partial attention results by their LSE.
 *
 * For context-parallel decoding the top-k entries of a row are split over P
 * owners (sglang PR 47013, Motivation: the DCP rework that gives each rank
 * ownership of its KV slots), each of which calls sparse_mla_attn on its own
 * entries (the others as -1) and gets the normalised output O_p and lse_p; the
 * same combination closes the split-K decode of sglang PR 39288, Motivation.
 * For every (row t, head h):
 *   lse = ln sum_p exp(lse_p),   out = sum_p exp(lse_p - lse) * O_p
 * A part with lse_p = -inf (no valid entry) weighs exactly 0 and its O_p is
 * not read; when every part is empty, out = 0 and lse = -inf.  fp32
 * arithmetic, out rounded to bf16 (nearest even).  With P = 1 the call
 * copies O_0 and lse_0.
 *
 * part_out        bf16 [P][T][H][512], contiguous, 16-byte aligned (e.g. the
 *                 gathered out tensors of P sparse_mla_attn calls).
 * part_lse        float32 [P][T][H] natural-log LSE, contiguous.
 * P, T, H         P >= 1, T >= 1, 1 <= H <= 128.
 * out             bf16 [T][H][512], 16-byte aligned; must not overlap the parts.
 * lse             float32 [T][H], or NULL.
 */
SMLA_API int sparse_mla_merge(const void* part_out, const float* part_lse, int P, int T, int H,
                     void* out, float* lse, hipStream_t stream);

/* Thread-local description of the last error returned on this thread ("" if none). */
SMLA_API const char* smla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H */
