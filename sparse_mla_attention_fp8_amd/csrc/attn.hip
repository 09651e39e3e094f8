// Sparse MLA attention over the fp8_ds_mla cache: split-top-k main kernel and
// the log-sum-exp merge of the splits.
//
// Semantics (sglang PR 47013, Motivation; sglang PR 39288, Root cause (1);
// vLLM PR 55277, Purpose): a query row attends over the valid entries of its
// top-k list (0 <= idx < num_slots); padding is never loaded and contributes
// exactly zero, so NaN-coded bytes in slot 0 cannot reach the output.
//
// Work decomposition: one 256-thread workgroup per (split, query row, group of
// 16 heads).  A split owns a contiguous range of the row's top-k buffer; it
// compacts the valid entries of its range into LDS, then walks them in chunks.
// With one split the workgroup writes the bf16 output and LSE itself; with
// several it writes (O unnormalised, m, l) partials that attn_merge combines.
#include "common.h"

namespace smla {
namespace {

constexpr int kThreads = 256;
constexpr int kHeadsPerGroup = 16;
constexpr int kChunk = 32;          // keys per inner step
constexpr int kMaxRange = 4096;     // top-k entries a split may own
constexpr int kTargetBlocks = 256;  // one workgroup per CU in the steady state

// OCP E4M3 code -> float32 (exact).  NaN codes give NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 7u;
  if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));
  if (e == 15u && m == 7u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Compacts the valid entries of idx[lo, hi) into list[], preserving order.
// Returns the count (same value in every thread).
__device__ int compact_valid(const int32_t* __restrict__ idx, int lo, int hi, int64_t num_slots,
                             int* list, int* wave_counts) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int base = lo; base < hi; base += kThreads) {
    const int k = base + tid;
    int v = -1;
    if (k < hi) v = idx[k];
    const bool ok = (k < hi) && v >= 0 && (int64_t)v < num_slots;
    const uint64_t mask = __ballot(ok);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wave_counts[wave] = __popcll(mask);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wave_counts[w];
    if (ok) list[off + before] = v;
    total += wave_counts[0] + wave_counts[1] + wave_counts[2] + wave_counts[3];
    __syncthreads();
  }
  return total;
}

template <int ROPE>
__global__ __launch_bounds__(kThreads) void attn_chunked_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots,
    const int32_t* __restrict__ idx, int64_t idx_stride, int W, int H, float sm_scale,
    int range, int splits, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int D = kLatent + ROPE;
  __shared__ int list[kMaxRange];
  __shared__ int wave_counts[4];
  __shared__ float qs[kHeadsPerGroup][D];
  __shared__ float ks[kChunk][D + 1];
  __shared__ float ps[kHeadsPerGroup][kChunk];

  const int split = blockIdx.x, t = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x;
  const int lo = split * range;
  const int hi = min(W, lo + range);
  const int n = compact_valid(idx + (int64_t)t * idx_stride, lo, hi, num_slots, list, wave_counts);

  // q of this head group as float (heads past H are zero)
  for (int i = tid; i < kHeadsPerGroup * D; i += kThreads) {
    const int h = i / D, d = i % D, hh = hg * kHeadsPerGroup + h;
    float v = 0.0f;
    if (hh < H) v = __uint_as_float((uint32_t)q[((int64_t)t * H + hh) * D + d] << 16);
    qs[h][d] = v;
  }

  const int h = tid >> 4;       // head owned in PV / softmax
  const int sub = tid & 15;     // 32 output dims [32*sub, 32*sub+32)
  float o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  for (int c0 = 0; c0 < n; c0 += kChunk) {
    const int nc = min(kChunk, n - c0);
    __syncthreads();  // previous chunk fully consumed (and qs ready on the first pass)
    // dequantise the chunk's rows into LDS
    for (int i = tid; i < nc * D; i += kThreads) {
      const int j = i / D, d = i % D;
      const uint8_t* row = cache + (int64_t)list[c0 + j] * kRowBytes;
      float v;
      if (d < kLatent) {
        const float sc = *reinterpret_cast<const float*>(row + kScaleOff + 4 * (d / kTile));
        v = e4m3_to_f32(row[d]) * sc;
      } else {
        const uint16_t b = *reinterpret_cast<const uint16_t*>(row + kRopeOff + 2 * (d - kLatent));
        v = __uint_as_float((uint32_t)b << 16);
      }
      ks[j][d] = v;
    }
    __syncthreads();
    // scores of keys sub and sub+16 for head h
    float s[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int j = sub + 16 * r;
      float acc = 0.0f;
      if (j < nc) {
        for (int d = 0; d < D; ++d) acc += qs[h][d] * ks[j][d];
        s[r] = acc * sm_scale;
      } else {
        s[r] = -INFINITY;
      }
    }
    float mc = fmaxf(s[0], s[1]);
    mc = fmaxf(mc, __shfl_xor(mc, 8, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 4, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 2, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 1, 16));
    const float m_new = fmaxf(m, mc);          // finite: the chunk has >= 1 valid key
    const float alpha = __expf(m - m_new);     // m = -inf on the first chunk -> 0
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int j = sub + 16 * r;
      const float p = (j < nc) ? __expf(s[r] - m_new) : 0.0f;
      ps[h][j] = p;
      psum += p;
    }
    psum += __shfl_xor(psum, 8, 16);
    psum += __shfl_xor(psum, 4, 16);
    psum += __shfl_xor(psum, 2, 16);
    psum += __shfl_xor(psum, 1, 16);
    l = l * alpha + psum;
    m = m_new;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] *= alpha;
    for (int j = 0; j < nc; ++j) {             // padding rows are never touched
      const float p = ps[h][j];
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] += p * ks[j][32 * sub + i];
    }
  }

  const int hh = hg * kHeadsPerGroup + h;
  if (hh >= H) return;
  if (splits == 1) {
    const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
    uint16_t* dst = out + ((int64_t)t * H + hh) * kLatent + 32 * sub;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const uint32_t pk = (uint32_t)f32_to_bf16_rne(o[i] * inv) |
                          ((uint32_t)f32_to_bf16_rne(o[i + 1] * inv) << 16);
      *reinterpret_cast<uint32_t*>(dst + i) = pk;
    }
    if (lse != nullptr && sub == 0) lse[(int64_t)t * H + hh] = (l > 0.0f) ? m + __logf(l) : -INFINITY;
  } else {
    const int64_t p = ((int64_t)t * splits + split) * H + hh;
    float* dst = part_o + p * kLatent + 32 * sub;
#pragma unroll
    for (int i = 0; i < 32; ++i) dst[i] = o[i];
    if (sub == 0) {
      part_ml[2 * p] = m;
      part_ml[2 * p + 1] = l;
    }
  }
}

// Combines split partials: M = max m_s, L = sum e^(m_s - M) l_s,
// O = sum e^(m_s - M) O_s / L, lse = M + ln L.  One 64-thread block per (row, head).
__global__ __launch_bounds__(64) void attn_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        int splits, int H,
                                                        uint16_t* __restrict__ out,
                                                        float* __restrict__ lse) {
  const int th = blockIdx.x;  // t * H + h
  const int t = th / H, hh = th % H;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[2 * (((int64_t)t * splits + s) * H + hh)]);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const int64_t p = ((int64_t)t * splits + s) * H + hh;
      const float ms = part_ml[2 * p];
      if (ms == -INFINITY) continue;  // empty split
      const float w = __expf(ms - M);
      L += w * part_ml[2 * p + 1];
      const float4* src = reinterpret_cast<const float4*>(part_o + p * kLatent + 8 * lane);
      const float4 a = src[0], b = src[1];
      acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
      acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
    }
  }
  const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = (uint32_t)f32_to_bf16_rne(acc[2 * i] * inv) |
            ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1] * inv) << 16);
  *reinterpret_cast<uint4*>(out + (int64_t)th * kLatent + 8 * lane) =
      make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse != nullptr && lane == 0) lse[th] = (L > 0.0f) ? M + __logf(L) : -INFINITY;
}

}  // namespace

AttnPlan plan_attn(int T, int H, int W, int rope_dim) {
  (void)rope_dim;
  AttnPlan p{};
  p.head_groups = (H + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int units = T * p.head_groups;
  const int max_splits = (W + kChunk - 1) / kChunk;
  int s = (kTargetBlocks + units - 1) / units;
  s = s < 1 ? 1 : (s > max_splits ? max_splits : s);
  const int min_s = (W + kMaxRange - 1) / kMaxRange;
  if (s < min_s) s = min_s;
  int range = (W + s - 1) / s;
  range = (range + kChunk - 1) / kChunk * kChunk;
  s = (W + range - 1) / range;
  p.splits = s;
  p.range = range;
  p.workspace = (s > 1) ? (size_t)T * s * H * (kLatent + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_attn(const uint16_t* q, const uint8_t* cache, int64_t num_slots,
                       const int32_t* idx, int64_t idx_stride, int W, int T, int H,
                       int rope_dim, float sm_scale, uint16_t* out, float* lse,
                       void* workspace, const AttnPlan& plan, hipStream_t stream) {
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (plan.splits > 1) {
    part_o = static_cast<float*>(workspace);
    part_ml = part_o + (size_t)T * plan.splits * H * kLatent;
  }
  const dim3 grid(plan.splits, T, plan.head_groups);
  if (rope_dim == 64)
    hipLaunchKernelGGL(attn_chunked_kernel<64>, grid, dim3(kThreads), 0, stream, q, cache,
                       num_slots, idx, idx_stride, W, H, sm_scale, plan.range, plan.splits, out,
                       lse, part_o, part_ml);
  else
    hipLaunchKernelGGL(attn_chunked_kernel<0>, grid, dim3(kThreads), 0, stream, q, cache,
                       num_slots, idx, idx_stride, W, H, sm_scale, plan.range, plan.splits, out,
                       lse, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(T * H), dim3(64), 0, stream, part_o, part_ml,
                     plan.splits, H, out, lse);
  return hipGetLastError();
}

}  // namespace smla
