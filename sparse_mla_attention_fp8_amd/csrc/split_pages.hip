// Re-paging of a pool of 256-token pages into a scratch of 64-token pages.
//
// Behaviour (sglang PR 39288, "zero-initialise the 64-token page-split
// scratch so masked candidates never gather NaN from slot 0", Root cause (2)
// and Modifications): the pool keeps 256-token pages while the reader wants
// 64-token pages, so each source page a step references is copied into four
// 64-token pages of a persistent scratch; pages the step does not reference
// are not copied.  The scratch is zero-filled once when it is allocated (the
// pages' fix), so its page 0 (slot 0) is finite whether or not source page 0
// is ever copied.  For every listed source page p (0 <= p < num_src_pages;
// other entries are ignored) and k = 0..3:
//   dst page 4p + k, bytes [0, 64 * row_bytes) = src page p, bytes
//   [64 * row_bytes * k, 64 * row_bytes * (k + 1))
// and nothing else is written.
//
// Mapping: one 256-thread workgroup per (listed page, quarter); 16-byte
// loads and stores, several in flight per thread.  HBM-bound: 2 x 64 x
// row_bytes per quarter.
#include "common.h"

namespace smla {
namespace {

constexpr int kSplitThreads = 256;
constexpr int kSplitUnroll = 4;

__global__ __launch_bounds__(kSplitThreads) void split_pages_kernel(
    const uint8_t* __restrict__ src, int64_t num_src_pages, int64_t src_page_stride,
    const int32_t* __restrict__ pages, uint8_t* __restrict__ dst, int64_t dst_page_stride,
    int row_bytes) {
  const int64_t item = blockIdx.x;             // (listed page, quarter)
  const int32_t p = pages[item >> 2];
  if (p < 0 || p >= num_src_pages) return;
  const int k = (int)(item & 3);
  // 64 rows: a multiple of 64 bytes whatever the row size (585-byte rows
  // make the 37,440-byte page), so every quarter is 16-byte aligned
  const int64_t bytes = 64 * (int64_t)row_bytes;
  const uint4* s = reinterpret_cast<const uint4*>(src + p * src_page_stride + k * bytes);
  uint4* d = reinterpret_cast<uint4*>(dst + (4 * (int64_t)p + k) * dst_page_stride);
  const int64_t n16 = bytes / 16;
  for (int64_t i0 = threadIdx.x; i0 < n16; i0 += kSplitThreads * kSplitUnroll) {
    uint4 v[kSplitUnroll];
#pragma unroll
    for (int u = 0; u < kSplitUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kSplitThreads;
      v[u] = i < n16 ? s[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kSplitUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * kSplitThreads;
      if (i < n16) d[i] = v[u];
    }
  }
}

}  // namespace

hipError_t launch_split_pages(const uint8_t* src, int64_t num_src_pages, int64_t src_page_stride,
                              const int32_t* pages, int64_t num_pages, uint8_t* dst,
                              int64_t dst_page_stride, int row_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(split_pages_kernel, dim3((unsigned)(4 * num_pages)), dim3(kSplitThreads), 0,
                     stream, src, num_src_pages, src_page_stride, pages, dst, dst_page_stride,
                     row_bytes);
  return hipGetLastError();
}

}  // namespace smla
