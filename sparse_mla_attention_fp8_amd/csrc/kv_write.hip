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
// form one 128-value tile, so the tile amax is a 16-lane DPP reduction.
// Lanes 0..7 also move the 128-byte RoPE tail.  Per kept row the kernel
// reads 1,152 B (1,024 without RoPE) and writes 656 B; the quantiser's
// arithmetic is kept short (one reciprocal per tile, three operations and a
// hardware conversion per value) so that a wavefront's chain of slot load,
// row load and store is not lengthened by it.
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


// Four codes of x[0..3] / scale, by IEEE division and the integer encoder.
__device__ __forceinline__ uint32_t encode4_exact(const float* x, float scale) {
  uint32_t p = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) p |= e4m3_rne_satfinite(x[i] / scale) << (8 * i);
  return p;
}

// DPP controls for a max over the 16 lanes of a row: swap neighbours, swap
// pairs, mirror each half-row, mirror the row.
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr uint32_t kBits448 = 0x43E00000u;   // 448.0f

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false));
}

// Four float32 values -> four e4m3 codes (byte i = value i) by the hardware
// conversion (round to nearest even).  It agrees with e4m3_rne_satfinite for
// every |v| <= 448; callers cap magnitudes at 448.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint16_t* __restrict__ kv_c, int64_t kv_c_stride,
    const uint16_t* __restrict__ k_pe, int64_t k_pe_stride, int rope_dim,
    const int64_t* __restrict__ slot_mapping, int64_t num_rows,
    uint8_t* __restrict__ cache, int64_t num_slots) {
  const int lane = threadIdx.x & 63;
  // wave-uniform row, so the slot id comes through one scalar load
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  // tile amax as an unsigned max of |x| bit patterns: the same order as the
  // float max for numbers, and a NaN anywhere in the tile makes amax NaN
  uint32_t am = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = max(am, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  am = dpp_max<kQuadXor1>(am);
  am = dpp_max<kQuadXor2>(am);
  am = dpp_max<kRowHalfMirror>(am);
  am = dpp_max<kRowMirror>(am);
  const float amax = __uint_as_float(am);

  const float scale = amax / 448.0f;  // IEEE float32 division (correctly rounded)
  uint32_t lo = 0u, hi = 0u;
  if (scale >= 0x1p-60f && scale <= 3.4028234663852886e38f) {
    // Fast path: the quotient x / scale from a reciprocal and one residual
    // correction (Markstein), q1 = fma(fma(-q0, scale, x), r, q0) with
    // r = fl32(1/scale) and q0 = fl32(x * r).  For a bf16 x and a float32
    // scale this is the IEEE quotient fl32(x / scale): an exhaustive run over
    // every float32 scale mantissa against every bf16 mantissa, in both
    // relative binades, found no difference, and the scale bound keeps every
    // intermediate normal wherever the quotient reaches the e4m3 grid.  The
    // sign of zero is taken from x.  Magnitudes are capped at 448 (the largest
    // code, to which every larger quotient saturates) before the hardware
    // conversion, which rounds to nearest even and gives the codes of
    // e4m3_rne_satfinite for every |v| <= 448.
    const float r = 1.0f / scale;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = __fmul_rn(x[i], r);
      const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, scale, x[i]), r, q0);
      const uint32_t mag = min(__float_as_uint(q1) & 0x7FFFFFFFu, kBits448);
      v[i] = __uint_as_float(mag | (__float_as_uint(x[i]) & 0x80000000u));
    }
    lo = pack4_e4m3(v[0], v[1], v[2], v[3]);
    hi = pack4_e4m3(v[4], v[5], v[6], v[7]);
  } else if (amax != 0.0f) {
    // tiny, huge or non-finite tiles: divide and encode exactly
    lo = encode4_exact(x, scale);
    hi = encode4_exact(x + 4, scale);
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
  // wave-uniform row, so the slot id comes through one scalar load
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
