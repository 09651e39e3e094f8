// Shared definitions of the HIP library (device and host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kRowBytes = 656;      // packed fp8_ds_mla row
constexpr int kLatent = 512;        // latent width = value width
constexpr int kTile = 128;          // quantisation tile
constexpr int kScaleOff = 512;      // 4 x float32 tile scales
constexpr int kRopeOff = 528;       // 64 x bf16 RoPE, or zeros for NoPE rows
constexpr int kNopeRowBytes = 528;  // bytes a NoPE reader needs

// Attention work decomposition, shared by the launch plan (host) and the kernels.
constexpr int kHeads = 16;          // heads per workgroup (MFMA N)
constexpr int kKeys = 64;           // keys per chunk (4 blocks of 16)
constexpr int kMaxRange = 2304;     // top-k entries one split may own (LDS index list)
constexpr int kTargetBlocks = 256;  // one workgroup per CU (LDS-bound occupancy)
constexpr int kFusedMaxSplits = 3;  // largest split count merged inside the main launch

// Internal launchers (return a hipError_t from the launch).
hipError_t launch_kv_write(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                           int64_t k_pe_stride, int rope_dim, const int64_t* slot_mapping,
                           int64_t num_rows, uint8_t* cache, int64_t num_slots,
                           hipStream_t stream);

hipError_t launch_kv_write_bf16(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                                int64_t k_pe_stride, int rope_dim, const int64_t* slot_mapping,
                                int64_t num_rows, uint16_t* cache, int64_t num_slots,
                                hipStream_t stream);

// Launch plan of the attention call; a pure function of the sizes, shared by
// the workspace query and the launch so the two always agree.
struct AttnPlan {
  int waves;         // wavefronts per workgroup of the fp8 kernel: 8 (64-key chunks, one
                     // workgroup per CU) or 4 (32-key chunks, two per CU) when the rows
                     // outnumber one round of eight-wavefront workgroups
  int head_groups;   // ceil(H / 16)
  int splits;        // split-top-k count per (row, head group)
  int range;         // top-k entries per split (multiple of the chunk size); 0: every split
                     // scans the whole row and keeps an equal share of its valid entries
  int64_t blocks;    // workgroups of the main launch (splits * T * head_groups)
  int fused;         // 1: the split of a (row, head group) that finishes last merges the
                     // row's partials inside the main launch (eight-wavefront plans of
                     // 2..kFusedMaxSplits splits); 0: a merge kernel follows
  size_t arrive_off; // byte offset in the workspace of the fused merge's arrival words
  size_t workspace;  // bytes of partial results and arrival words (0 when splits == 1)
};
AttnPlan plan_attn(int T, int H, int topk_capacity, int rope_dim);

hipError_t launch_attn(const uint16_t* q, const uint8_t* cache, int64_t num_slots,
                       const int32_t* idx, int64_t idx_stride, int W, int T, int H,
                       int rope_dim, float sm_scale, uint16_t* out, float* lse,
                       void* workspace, const AttnPlan& plan, hipStream_t stream);

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* cache, int64_t num_slots,
                            const int32_t* idx, int64_t idx_stride, int W, int T, int H,
                            int rope_dim, float sm_scale, uint16_t* out, float* lse, void* workspace,
                            const AttnPlan& plan, hipStream_t stream);

hipError_t launch_gather_upconvert(const uint8_t* cache, int64_t num_slots, int rope_dim,
                                   const int64_t* slots, int64_t n, uint16_t* dst,
                                   int64_t dst_stride, hipStream_t stream);

hipError_t launch_split_pages(const uint8_t* src, int64_t num_src_pages, int64_t src_page_stride,
                              const int32_t* pages, int64_t num_pages, uint8_t* dst,
                              int64_t dst_page_stride, int row_bytes, hipStream_t stream);

hipError_t launch_merge(const uint16_t* part_out, const float* part_lse, int P, int64_t rows,
                        uint16_t* out, float* lse, hipStream_t stream);

// Gather-only measurement kernel (smla_gather_rows_probe).
int64_t gather_probe_max_rows();
hipError_t launch_gather_probe(const uint8_t* cache, int64_t num_slots, int rope_dim, const int32_t* slots,
                               int64_t n, uint32_t* sink, hipStream_t stream);

// Scratch of the allocation-free attention entry point: a device array of
// kNoallocScratchBytes per GPU; *out = its address on the stream's device.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** out);

}  // namespace smla
