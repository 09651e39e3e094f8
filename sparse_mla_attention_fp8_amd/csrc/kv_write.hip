// KV-row writer: bf16 latent (+ RoPE) rows -> 656-byte fp8_ds_mla cache rows.
//
// Behaviour (sglang PR 47013, "zero-RoPE MLA KV writer skips reserved slot
// 0", Summary / Modifications; vLLM PR 55277, Purpose (1)):
//   * a row aimed at slot 0 (reserved for padding), a negative slot or one past
//     the cache is dropped before any of its input is read;
//   * per 128-value tile: scale = fp32(amax / 448), code = e4m3(fp32(x/scale))
//     with round-to-nearest-even and saturation at 448; amax == 0 gives scale 0
//     and zero codes;
//   * bytes 528..655 get the 64 bf16 RoPE values, or zeros for NoPE rows.
//
// Mapping: one 64-lane wavefront per row.  Lane l owns latent values
// 8l..8l+7 (one 16-byte load, one 8-byte store); the 16 lanes of a DPP row
// form one 128-value tile, so the tile amax is a 16-lane reduction.  Lanes
// 0..7 also move the 128-byte RoPE tail.  The kernel is HBM-bound: per kept
// row it reads 1,152 B (1,024 without RoPE) and writes 656 B.
#include "common.h"

namespace smla {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts per 256-thread block

// float32 -> OCP E4M3 code, round to nearest even, saturating to +-448, sign of
// zero kept.  Integer-exact, so the result does not depend on conversion
// hardware modes.
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN stays NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |v| >= 448: every such value rounds to or past 448
  if (a < 0x3C800000u) {                      // |v| < 2^-6: subnormal grid of 2^-9
    const float t = __uint_as_float(a) * 512.0f;   // exact power-of-two scaling, t < 8
    return sign | (uint32_t)__builtin_rintf(t);     // 8 carries into the smallest normal
  }
  const uint32_t e = (a >> 23) - 120u;        // biased e4m3 exponent, 1..15
  const uint32_t mant = (a >> 20) & 7u;
  const uint32_t rem = a & 0xFFFFFu;           // the 20 dropped mantissa bits
  const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & mant);
  uint32_t code = (e << 3) + mant + (up & 1u); // a mantissa carry bumps the exponent
  code = code > 0x7Eu ? 0x7Eu : code;
  return sign | code;
}

__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint16_t* __restrict__ kv_c, int64_t kv_c_stride,
    const uint16_t* __restrict__ k_pe, int64_t k_pe_stride, int rope_dim,
    const int64_t* __restrict__ slot_mapping, int64_t num_rows,
    uint8_t* __restrict__ cache, int64_t num_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= num_rows) return;
  const int64_t slot = slot_mapping[row];
  if (slot <= 0 || slot >= num_slots) return;  // dropped: inputs never read

  uint8_t* dst = cache + slot * (int64_t)kRowBytes;

  // RoPE tail first: lanes 0..7 move 16 bytes each (or write zeros).
  if (lane < 8) {
    uint4 r = make_uint4(0u, 0u, 0u, 0u);
    if (rope_dim == 64) r = *reinterpret_cast<const uint4*>(k_pe + row * k_pe_stride + lane * 8);
    *reinterpret_cast<uint4*>(dst + kRopeOff + lane * 16) = r;
  }

  const uint4 raw = *reinterpret_cast<const uint4*>(kv_c + row * kv_c_stride + lane * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  // 16-lane (one tile) max reduction
  amax = fmaxf(amax, __shfl_xor(amax, 8, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 16));

  const float scale = amax / 448.0f;  // IEEE float32 division (correctly rounded)
  uint32_t lo = 0u, hi = 0u;
  if (amax != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_rne_satfinite(x[i] / scale) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_rne_satfinite(x[4 + i] / scale) << (8 * i);
  }
  *reinterpret_cast<uint2*>(dst + lane * 8) = make_uint2(lo, hi);
  if ((lane & 15) == 0)
    *reinterpret_cast<float*>(dst + kScaleOff + 4 * (lane >> 4)) = scale;
}

// BF16 cache rows (sglang PR 47013, Speed Tests: rows of 512 bf16 values):
// row = bf16 [512 + rope_dim], written as is, with the same slot rule.  One
// wavefront per row: lane l moves latent values 8l..8l+7, lanes 0..7 the RoPE
// values.
__global__ __launch_bounds__(64 * kRowsPerBlock) void kv_write_bf16_kernel(
    const uint16_t* __restrict__ kv_c, int64_t kv_c_stride, const uint16_t* __restrict__ k_pe,
    int64_t k_pe_stride, int rope_dim, const int64_t* __restrict__ slot_mapping, int64_t num_rows,
    uint16_t* __restrict__ cache, int64_t num_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= num_rows) return;
  const int64_t slot = slot_mapping[row];
  if (slot <= 0 || slot >= num_slots) return;   // dropped before any input load
  uint16_t* dst = cache + slot * (int64_t)(kLatent + rope_dim);
  const uint4 v = reinterpret_cast<const uint4*>(kv_c + row * kv_c_stride)[lane];
  uint4 pe = make_uint4(0, 0, 0, 0);
  if (rope_dim != 0 && lane < 8) pe = reinterpret_cast<const uint4*>(k_pe + row * k_pe_stride)[lane];
  reinterpret_cast<uint4*>(dst)[lane] = v;
  if (rope_dim != 0 && lane < 8) reinterpret_cast<uint4*>(dst + kLatent)[lane] = pe;
}

}  // namespace

hipError_t launch_kv_write_bf16(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                                int64_t k_pe_stride, int rope_dim, const int64_t* slot_mapping,
                                int64_t num_rows, uint16_t* cache, int64_t num_slots,
                                hipStream_t stream) {
  if (num_rows == 0) return hipSuccess;
  const int64_t blocks = (num_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(kv_write_bf16_kernel, dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0,
                     stream, kv_c, kv_c_stride, k_pe, k_pe_stride, rope_dim, slot_mapping, num_rows,
                     cache, num_slots);
  return hipGetLastError();
}

hipError_t launch_kv_write(const uint16_t* kv_c, int64_t kv_c_stride, const uint16_t* k_pe,
                           int64_t k_pe_stride, int rope_dim, const int64_t* slot_mapping,
                           int64_t num_rows, uint8_t* cache, int64_t num_slots,
                           hipStream_t stream) {
  if (num_rows == 0) return hipSuccess;
  const int64_t blocks = (num_rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv_c,
                     kv_c_stride, k_pe, k_pe_stride, rope_dim, slot_mapping, num_rows, cache,
                     num_slots);
  return hipGetLastError();
}

}  // namespace smla
