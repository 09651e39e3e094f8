// Standalone merge of partial attention results by their log-sum-exp.
//
// When the top-k entries of a query row are split over P owners (the context-
// parallel decode ranks that sglang PR 47013, Motivation, names as the DCP
// rework, or the split-K decode kernel of sglang PR 39288, Motivation), each
// owner attends over its own entries and returns the normalised output O_p
// (bf16) and the natural-log LSE lse_p.  The full result is
//   lse = ln sum_p exp(lse_p),   O = sum_p exp(lse_p - lse) * O_p,
// and parts with lse_p = -inf (no valid entry) weigh nothing; when every part
// is empty, O = 0 and lse = -inf.
//
// Mapping: one 64-lane wavefront per (row, head); lane l owns dims 8l..8l+7
// (one 16-byte load per part, one 16-byte store).  The parts are taken eight
// at a time with a running maximum, so a group's loads are all in flight
// together.  HBM-bound: per (row, head) it reads P * (1,024 + 4) bytes and
// writes 1,024 (+ 4).
#include "common.h"

namespace smla {
namespace {

constexpr int kMergeRowsPerBlock = 4;   // 4 wavefronts per 256-thread block
constexpr int kGroup = 8;               // parts whose loads are in flight together

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void add_bf16x8(float* acc, float w, const uint4 v) {
  const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += w * __uint_as_float(p[i] << 16);
    acc[2 * i + 1] += w * __uint_as_float(p[i] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(64 * kMergeRowsPerBlock) void merge_partials_kernel(
    const uint16_t* __restrict__ part_out, const float* __restrict__ part_lse, int P,
    int64_t rows, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kMergeRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // t * H + h (wave-uniform)
  if (r >= rows) return;
  const uint4* src = reinterpret_cast<const uint4*>(part_out + r * kLatent) + lane;
  const int64_t pstride = rows * (kLatent / 8);   // uint4 units between parts
  // Online over groups of kGroup parts: every load of a group is issued before
  // any is used; the running max M and sum S rescale when M grows.
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  float M = -INFINITY, S = 0.0f;
  for (int p0 = 0; p0 < P; p0 += kGroup) {
    float l[kGroup];
    uint4 v[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const bool in = p0 + k < P;
      l[k] = in ? part_lse[(int64_t)(p0 + k) * rows + r] : -INFINITY;
      v[k] = in ? src[(int64_t)(p0 + k) * pstride] : make_uint4(0, 0, 0, 0);
    }
    float gm = M;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) gm = fmaxf(gm, l[k]);
    if (gm == -INFINITY) continue;                  // nothing valid yet
    const float c = expf(M - gm);                   // 0 while M is -inf
    S *= c;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= c;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      // an empty part (lse -inf) weighs exactly 0 and its output is never used
      if (l[k] != -INFINITY) {
        const float w = expf(l[k] - gm);
        S += w;
        add_bf16x8(acc, w, v[k]);
      }
    }
    M = gm;
  }
  float L = -INFINITY;
  uint32_t pk[4] = {0, 0, 0, 0};
  if (M != -INFINITY) {
    L = M + logf(S);
    const float inv = 1.0f / S;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pk[i] = (uint32_t)bf16_rne(acc[2 * i] * inv) | ((uint32_t)bf16_rne(acc[2 * i + 1] * inv) << 16);
  }
  reinterpret_cast<uint4*>(out + r * kLatent)[lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse != nullptr && lane == 0) lse[r] = L;
}

}  // namespace

hipError_t launch_merge(const uint16_t* part_out, const float* part_lse, int P, int64_t rows,
                        uint16_t* out, float* lse, hipStream_t stream) {
  const int64_t blocks = (rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock;
  hipLaunchKernelGGL(merge_partials_kernel, dim3((unsigned)blocks), dim3(64 * kMergeRowsPerBlock),
                     0, stream, part_out, part_lse, P, rows, out, lse);
  return hipGetLastError();
}

}  // namespace smla
