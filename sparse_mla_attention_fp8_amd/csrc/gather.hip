// Gather + upconvert: listed fp8_ds_mla cache rows -> a bf16 workspace of
// 576-wide rows, the form a chunked-context (prefill) reader consumes.
//
// Behaviour (vLLM PR 55277, "Support NoPE sparse MLA (GLM-5.3-Flash) on the
// FlashInfer SM120 backend", Purpose (1) and the review comment on the
// gather: with pe_dim == 0 the reader must see exact zeros in columns 512..575,
// never stale cache bytes):
//   for each i with 0 <= slots[i] < num_slots, row = cache[slots[i]]:
//     dst[i][e]       = bf16(fp32(e4m3(code[e]) * scale[e / 128]))   e < 512
//     dst[i][512 + r] = RoPE value r (rope_dim 64) or +0 (rope_dim 0; the
//                       row's bytes 528..655 are not read then)
//   any other entry (negative or >= num_slots) gives an all-zero row.
// The dequantised value is rounded once to fp32 (the precision of the stored
// scale), then to bf16, both to nearest even.
//
// Mapping: one 64-lane wavefront per 2 rows, whose loads are all issued
// before any is used.  Lane l owns latent values 8l..8l+7 of a row: one 8-byte
// code load, its tile's scale, one 16-byte store.  Lanes 0..7 also move the
// 128-byte RoPE tail (or store its zeros).  HBM-bound: per row it reads
// 8 + 528 (+ 128 with RoPE) bytes and writes 1,152.
#include "common.h"

namespace smla {
namespace {

constexpr int kGatherWaves = 4;          // wavefronts per 256-thread block
constexpr int kRowsPerWave = 2;          // rows per wavefront, loaded together
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(64 * kGatherWaves) void gather_upconvert_kernel(
    const uint8_t* __restrict__ cache, int64_t num_slots, int rope_dim,
    const int64_t* __restrict__ slots, int64_t n, uint16_t* __restrict__ dst, int64_t dst_stride) {
  const int lane = threadIdx.x & 63;
  // wave-uniform rows, so the slot ids come through scalar loads
  const int64_t i0 = ((int64_t)blockIdx.x * kGatherWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * kRowsPerWave;
  if (i0 >= n) return;
  // all of this wavefront's loads first, so kRowsPerWave rows are in flight at once
  bool ok[kRowsPerWave];
  uint2 codes[kRowsPerWave];
  float scale[kRowsPerWave];
  uint4 tail[kRowsPerWave];
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int64_t i = i0 + k;
    const int64_t slot = i < n ? slots[i] : -1;
    ok[k] = slot >= 0 && slot < num_slots;
    codes[k] = make_uint2(0, 0);
    scale[k] = 0.0f;
    tail[k] = make_uint4(0, 0, 0, 0);
    if (ok[k]) {
      const uint8_t* row = cache + slot * (int64_t)kRowBytes;
      codes[k] = reinterpret_cast<const uint2*>(row)[lane];
      scale[k] = reinterpret_cast<const float*>(row + kScaleOff)[lane >> 4];
      if (rope_dim != 0 && lane < 8) tail[k] = reinterpret_cast<const uint4*>(row + kRopeOff)[lane];
    }
  }
#pragma unroll
  for (int k = 0; k < kRowsPerWave; ++k) {
    const int64_t i = i0 + k;
    if (i >= n) break;
    uint16_t* drow = dst + i * dst_stride;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (ok[k]) {
      // the hardware fp8 -> f32 conversion is exact for every e4m3 code
      // (NaN codes give NaN); the product is rounded once to f32
      const int c[2] = {(int)codes[k].x, (int)codes[k].y};
      uint32_t pk[4];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const f2 ab = __builtin_amdgcn_cvt_pk_f32_fp8(c[w], false);
        const f2 cd = __builtin_amdgcn_cvt_pk_f32_fp8(c[w], true);
        pk[2 * w] = bf16_rne_bits(ab[0] * scale[k]) | (bf16_rne_bits(ab[1] * scale[k]) << 16);
        pk[2 * w + 1] = bf16_rne_bits(cd[0] * scale[k]) | (bf16_rne_bits(cd[1] * scale[k]) << 16);
      }
      o = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    reinterpret_cast<uint4*>(drow)[lane] = o;
    if (lane < 8) reinterpret_cast<uint4*>(drow + kLatent)[lane] = tail[k];
  }
}

}  // namespace

hipError_t launch_gather_upconvert(const uint8_t* cache, int64_t num_slots, int rope_dim,
                                   const int64_t* slots, int64_t n, uint16_t* dst,
                                   int64_t dst_stride, hipStream_t stream) {
  constexpr int64_t kRowsPerBlock = kGatherWaves * kRowsPerWave;
  const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(gather_upconvert_kernel, dim3((unsigned)blocks), dim3(64 * kGatherWaves), 0,
                     stream, cache, num_slots, rope_dim, slots, n, dst, dst_stride);
  return hipGetLastError();
}

}  // namespace smla
