// Sparse MLA attention over the fp8_ds_mla cache: split-top-k main kernel on
// CDNA4 matrix cores, and the log-sum-exp merge of the splits.
//
// Semantics (sglang PR 47013, Motivation; sglang PR 39288, Root cause (1);
// vLLM PR 55277, Purpose): a query row attends over the valid entries of its
// top-k list (0 <= idx < num_slots).  Padding is never gathered and carries an
// exact zero weight, so NaN-coded bytes in slot 0 cannot reach the output.
//
// Work decomposition.  One 256-thread workgroup (4 wavefronts) per
// (split, query row, group of 16 heads).  A split owns a contiguous range of
// the row's top-k buffer; the workgroup compacts the valid entries of its
// range into LDS and walks them in chunks of 64 keys:
//
//   gather  Each chunk's 64 rows (656 B, or the 528 B a NoPE reader needs)
//           are copied HBM -> LDS with direct-to-LDS 16-byte loads, once per
//           chunk and shared by all heads; a 3-stage ring keeps two chunks in
//           flight while one is computed.  Entries past the valid count of the
//           last chunk get a copy of the chunk's first valid row (so every LDS
//           operand is finite) and a weight that is exactly zero by select.
//   QK^T    Wavefront w scores keys 16w..16w+15 against all 16 heads:
//           S^T = K Q^T on v_mfma_f32_16x16x32_fp8_fp8, fed directly with the
//           cached e4m3 codes.  q (bf16) is split exactly into an e4m3 high
//           part and an e4m3 residual after a power-of-two prescale, so two
//           fp8 products give the bf16 q to within e4m3 subnormal flushing.
//           Each 128-wide tile accumulates separately and is scaled by its
//           fp32 tile scale; the RoPE part (bf16) uses the bf16 MFMA.
//   softmax Base-2 online softmax: block maxima and sums cross the four
//           wavefronts through LDS together with p * scale_tile.
//   P.V     Wavefront w owns latent tile w (128 dims): O^T = V^T P^T with the
//           e4m3 codes as V (transposed in registers from 8-byte LDS reads by
//           byte permutes) and P * scale_tile split into e4m3 high + residual
//           after a per-head power-of-two normalisation.
//
// With one split the workgroup writes the bf16 output and LSE; with several it
// writes (O unnormalised fp32, m, l) partials that attn_merge combines.  m is
// kept in log2 units throughout.
#include "common.h"

namespace smla {
namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 16;          // heads per workgroup (MFMA N)
constexpr int kKeys = 64;           // keys per chunk (4 blocks of 16)
constexpr int kMaxRange = 2304;     // top-k entries one split may own
constexpr int kTargetBlocks = 256;  // one workgroup per CU (LDS-bound occupancy)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <int ROPE>
struct Geo {
  static constexpr int D = kLatent + ROPE;          // q width
  static constexpr int RB = ROPE ? 656 : 528;       // bytes staged per row
  static constexpr int NSEG = RB / 16;              // 16-byte segments per row
  static constexpr int STAGE = kKeys * RB;          // bytes per stage
  // a chunk is NSEG direct-to-LDS instructions of 64 x 16 B, dealt round-robin
  // to the 4 wavefronts; wavefront 0 takes the extra one
  static constexpr int CNT0 = (NSEG + 3) / 4;
  static constexpr int CNT = NSEG / 4;
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14])
constexpr int vm_lgkm0_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }
constexpr int kLgkm0 = vm_lgkm0_wait(63);

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane.
// Issued as inline asm so the compiler adds no waits of its own for it: the
// pipeline below accounts for these loads with explicit vmcnt waits.  m0 (the
// LDS base operand) is saved and restored around the load.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// All waves' LDS writes visible to every wave of the workgroup (no wait on global loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// Own direct-to-LDS loads down to N outstanding, LDS ops drained, then a workgroup barrier.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  __builtin_amdgcn_s_waitcnt(vm_lgkm0_wait(N));
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float exp2_pow(int e) {  // 2^e for e in [-126, 127]
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// x (4 floats) -> e4m3 high part (packed dword) and e4m3 residual (packed dword)
__device__ __forceinline__ void split_e4m3(float x0, float x1, float x2, float x3,
                                           uint32_t& hi, uint32_t& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const f2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - b01[0], x1 - b01[1], 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b23[0], x3 - b23[1], l, true);
  hi = (uint32_t)h;
  lo = (uint32_t)l;
}

// 4x4 byte transpose: in a_i byte j -> out b_j byte i
__device__ __forceinline__ void tr4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                      uint32_t& b0, uint32_t& b1, uint32_t& b2, uint32_t& b3) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x06020400u);
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030501u);
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x06020400u);
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030501u);
  b0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  b2 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  b1 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  b3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

__device__ __forceinline__ long pack64(uint32_t lo, uint32_t hi) {
  return (long)(((uint64_t)hi << 32) | lo);
}

// Compacts the valid entries of idx[lo, hi) into list[] in order; returns the count.
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
__global__ __launch_bounds__(kThreads, 1) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots,
    const int32_t* __restrict__ idx, int64_t idx_stride, int W, int H, float sm_scale_log2,
    int range, int splits, int head_groups, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  using G = Geo<ROPE>;
  constexpr int D = G::D, RB = G::RB, NSEG = G::NSEG;

  __shared__ __align__(16) uint8_t st0[G::STAGE];
  __shared__ __align__(16) uint8_t st1[G::STAGE];
  __shared__ __align__(16) uint8_t st2[G::STAGE];
  __shared__ int slot_list[kMaxRange];
  __shared__ __align__(16) float4 pex[4][4][64];   // [tile][block][lane] -> p*scale_tile, keys 4g+r
  __shared__ float mex[4][kHeads];                  // block max (log2 units)
  __shared__ float lex[4][kHeads];                  // block sum
  __shared__ int wave_counts[4];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values are made visibly uniform so that every barrier sits on
  // scalar control flow
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  int b = blockIdx.x;
  const int split = b % splits;
  b /= splits;
  const int hg = b % head_groups;
  const int t = b / head_groups;

  // ---- q fragments of head n16 (issued before the index scan) ------------
  const int head = hg * kHeads + n16;
  const bool hvalid = head < H;
  const uint16_t* qrow = q + ((int64_t)t * H + (hvalid ? head : 0)) * D;
  uint4 qraw[16];   // k-step 2s+h: dims 64s + 16g + 8h + [0, 8)
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qraw[2 * s] = *reinterpret_cast<const uint4*>(qrow + 64 * s + 16 * g);
    qraw[2 * s + 1] = *reinterpret_cast<const uint4*>(qrow + 64 * s + 16 * g + 8);
  }
  uint4 qpe_raw[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if (ROPE) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      qpe_raw[u] = *reinterpret_cast<const uint4*>(qrow + kLatent + 32 * u + 8 * g);
  }

  const int lo_k = split * range;
  const int hi_k = min(W, lo_k + range);
  const int n = __builtin_amdgcn_readfirstlane(
      compact_valid(idx + (int64_t)t * idx_stride, lo_k, hi_k, num_slots, slot_list, wave_counts));
  const int nch = (n + kKeys - 1) / kKeys;

  // ---- q -> e4m3 high + residual, prescaled by a power of two -------------
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w4[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w4[j] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w4[j] & 0xFFFF0000u)));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  // amax * 2^a < 256 with a = 134 - biased exponent of amax
  int qe = 0;
  if (amax > 0.0f) {
    qe = 134 - (int)((__float_as_uint(amax) >> 23) & 0xFF);
    qe = qe > 126 ? 126 : (qe < -126 ? -126 : qe);
  }
  const float qscale = exp2_pow(qe);
  const float qinv = exp2_pow(-qe);
  long qhi[16], qlo[16];
  if (!hvalid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) qraw[i] = make_uint4(0, 0, 0, 0);
    qpe_raw[0] = qpe_raw[1] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w4[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w4[j] << 16) * qscale;
      x[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u) * qscale;
    }
    uint32_t h0, l0, h1, l1;
    split_e4m3(x[0], x[1], x[2], x[3], h0, l0);
    split_e4m3(x[4], x[5], x[6], x[7], h1, l1);
    qhi[i] = pack64(h0, h1);
    qlo[i] = pack64(l0, l1);
  }
  bf16x8 qpe[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) qpe[u] = __builtin_bit_cast(bf16x8, qpe_raw[u]);

  // ---- gather geometry: instruction i = wave + 4j covers flat segments 64i + lane
  const int my_cnt = wave == 0 ? G::CNT0 : G::CNT;
  int seg_row[G::CNT0];
  int seg_off[G::CNT0];
#pragma unroll
  for (int j = 0; j < G::CNT0; ++j) {
    const int f = 64 * (wave + 4 * j) + lane;
    seg_row[j] = f / NSEG;
    seg_off[j] = (f % NSEG) * 16;
  }
  auto issue = [&](uint32_t stage, int c) {
    const int base = c * kKeys;
    const int nv = min(kKeys, n - base);
    const int first = slot_list[base];
#pragma unroll
    for (int j = 0; j < G::CNT0; ++j) {
      if (j < my_cnt) {
        const int r = seg_row[j];
        const int slot = r < nv ? slot_list[base + r] : first;
        const uint8_t* src = cache + (int64_t)slot * kRowBytes + seg_off[j];
        dma16(src, stage + 1024u * (uint32_t)(wave + 4 * j));
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f4 oacc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) oacc[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const uint8_t* stg, int c) {
    const int nv = min(kKeys, n - c * kKeys);
    // ---------------- QK^T for keys 16*wave + [0, 16) ----------------
    const uint8_t* krow = stg + (16 * wave + n16) * RB;
    f4 acc[4];
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) acc[tl] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(krow + 64 * s + 16 * g);
      const int tl = s >> 1;
      acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pack64(a.x, a.y), qhi[2 * s], acc[tl], 0, 0, 0);
      acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pack64(a.x, a.y), qlo[2 * s], acc[tl], 0, 0, 0);
      acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pack64(a.z, a.w), qhi[2 * s + 1], acc[tl], 0, 0, 0);
      acc[tl] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(pack64(a.z, a.w), qlo[2 * s + 1], acc[tl], 0, 0, 0);
    }
    f4 accr = f4{0.0f, 0.0f, 0.0f, 0.0f};
    if (ROPE) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kRopeOff + 64 * u + 16 * g);
        accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qpe[u], accr, 0, 0, 0);
      }
    }
    // lane (head n16, g) holds keys 16*wave + 4g + r, r = 0..3
    float4 sc[4];
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * wave + 4 * g + r;
      sc[r] = *reinterpret_cast<const float4*>(stg + key * RB + kScaleOff);
      const float dot = qinv * (sc[r].x * acc[0][r] + sc[r].y * acc[1][r] +
                                sc[r].z * acc[2][r] + sc[r].w * acc[3][r]) + accr[r];
      sv[r] = key < nv ? dot * sm_scale_log2 : -INFINITY;
    }
    float mb = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    float p[4];
    float lb = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = (16 * wave + 4 * g + r < nv) ? __builtin_amdgcn_exp2f(sv[r] - mb) : 0.0f;
      lb += p[r];
    }
    lb += __shfl_xor(lb, 16);
    lb += __shfl_xor(lb, 32);
    pex[0][wave][lane] = make_float4(p[0] * sc[0].x, p[1] * sc[1].x, p[2] * sc[2].x, p[3] * sc[3].x);
    pex[1][wave][lane] = make_float4(p[0] * sc[0].y, p[1] * sc[1].y, p[2] * sc[2].y, p[3] * sc[3].y);
    pex[2][wave][lane] = make_float4(p[0] * sc[0].z, p[1] * sc[1].z, p[2] * sc[2].z, p[3] * sc[3].z);
    pex[3][wave][lane] = make_float4(p[0] * sc[0].w, p[1] * sc[1].w, p[2] * sc[2].w, p[3] * sc[3].w);
    if (g == 0) {
      mex[wave][n16] = mb;
      lex[wave][n16] = lb;
    }
    lds_barrier();

    // ---------------- softmax state ----------------
    float mbs[4], fb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) mbs[k] = mex[k][n16];
    const float m_new = fmaxf(fmaxf(fmaxf(m_run, mbs[0]), mbs[1]), fmaxf(mbs[2], mbs[3]));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      fb[k] = __builtin_amdgcn_exp2f(mbs[k] - m_new);       // empty block: -inf -> 0
      lsum += fb[k] * lex[k][n16];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;

    // ---------------- P.V for latent tile `wave` ----------------
    float x[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float4 v0 = pex[wave][2 * s][lane];
      const float4 v1 = pex[wave][2 * s + 1][lane];
      const float f0 = fb[2 * s], f1 = fb[2 * s + 1];
      x[s][0] = v0.x * f0; x[s][1] = v0.y * f0; x[s][2] = v0.z * f0; x[s][3] = v0.w * f0;
      x[s][4] = v1.x * f1; x[s][5] = v1.y * f1; x[s][6] = v1.z * f1; x[s][7] = v1.w * f1;
    }
    float nm = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) nm = fmaxf(nm, x[s][e]);
    nm = fmaxf(nm, __shfl_xor(nm, 16));
    nm = fmaxf(nm, __shfl_xor(nm, 32));
    // power of two N2 >= nm; operands scaled into [0, 256]
    int ne = 0;
    if (nm > 0.0f) {
      const uint32_t bits = __float_as_uint(nm);
      ne = (int)((bits >> 23) & 0xFF) - 127 + ((bits & 0x7FFFFF) ? 1 : 0);
      ne = ne > 119 ? 119 : (ne < -126 ? -126 : ne);
    }
    const float inv = exp2_pow(8 - ne);
    const float post = exp2_pow(ne - 8);
    long bhi[2], blo[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint32_t h0, l0, h1, l1;
      split_e4m3(x[s][0] * inv, x[s][1] * inv, x[s][2] * inv, x[s][3] * inv, h0, l0);
      split_e4m3(x[s][4] * inv, x[s][5] * inv, x[s][6] * inv, x[s][7] * inv, h1, l1);
      bhi[s] = pack64(h0, h1);
      blo[s] = pack64(l0, l1);
    }
    f4 tacc[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) tacc[cc] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint2 v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 32 * s + 16 * (e >> 2) + 4 * g + (e & 3);
        v[e] = *reinterpret_cast<const uint2*>(stg + key * RB + 128 * wave + 8 * n16);
      }
      uint32_t lo[8], hi[8];
      tr4x4(v[0].x, v[1].x, v[2].x, v[3].x, lo[0], lo[1], lo[2], lo[3]);
      tr4x4(v[4].x, v[5].x, v[6].x, v[7].x, hi[0], hi[1], hi[2], hi[3]);
      tr4x4(v[0].y, v[1].y, v[2].y, v[3].y, lo[4], lo[5], lo[6], lo[7]);
      tr4x4(v[4].y, v[5].y, v[6].y, v[7].y, hi[4], hi[5], hi[6], hi[7]);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const long a = pack64(lo[cc], hi[cc]);
        tacc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, bhi[s], tacc[cc], 0, 0, 0);
        tacc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, blo[s], tacc[cc], 0, 0, 0);
      }
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[cc][r] = oacc[cc][r] * alpha + tacc[cc][r] * post;
  };

  // ---- pipeline: chunk c lives in stage c % 3; two chunks in flight -------
  const uint32_t a0 = lds_addr(st0), a1 = lds_addr(st1), a2 = lds_addr(st2);
  // Every compiler-visible load (q) is complete before the pipeline starts, so
  // the compiler has no reason to emit a vmcnt wait of its own in the loop
  // (it does not count the inline-asm gathers; a wait of its own there would
  // drain the whole pipeline).
  __builtin_amdgcn_s_waitcnt(0);
  if (nch > 0) issue(a0, 0);
  if (nch > 1) issue(a1, 1);
  auto step = [&](const uint8_t* cur, uint32_t nxt2, int c) {
    if (c + 1 < nch) {
      if (wave == 0) vm_barrier<G::CNT0>(); else vm_barrier<G::CNT>();
    } else {
      vm_barrier<0>();
    }
    if (c + 2 < nch) issue(nxt2, c + 2);
    compute(cur, c);
  };
  for (int c = 0; c < nch; c += 3) {
    step(st0, a2, c);
    if (c + 1 < nch) step(st1, a0, c + 1);
    if (c + 2 < nch) step(st2, a1, c + 2);
  }

  // ---- epilogue ----------------------------------------------------------
  if (!hvalid) return;
  const int dim0 = 128 * wave + 32 * g;   // lane's dims: dim0 + 8r + c
  if (splits == 1) {
    const float il = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    uint16_t* dst = out + ((int64_t)t * H + head) * kLatent + dim0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        pk[k] = (uint32_t)f32_to_bf16_rne(oacc[2 * k][r] * il) |
                ((uint32_t)f32_to_bf16_rne(oacc[2 * k + 1][r] * il) << 16);
      *reinterpret_cast<uint4*>(dst + 8 * r) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    if (lse != nullptr && wave == 0 && g == 0)
      lse[(int64_t)t * H + head] = l_run > 0.0f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const int64_t p = ((int64_t)t * splits + split) * H + head;
    float* dst = part_o + p * kLatent + dim0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4*>(dst + 8 * r) = make_float4(oacc[0][r], oacc[1][r], oacc[2][r], oacc[3][r]);
      *reinterpret_cast<float4*>(dst + 8 * r + 4) = make_float4(oacc[4][r], oacc[5][r], oacc[6][r], oacc[7][r]);
    }
    if (wave == 0 && g == 0) {
      part_ml[2 * p] = m_run;
      part_ml[2 * p + 1] = l_run;
    }
  }
}

// Combines split partials (m in log2 units): M = max m_s, L = sum 2^(m_s - M) l_s,
// O = sum 2^(m_s - M) O_s / L, lse = (M + log2 L) ln 2.  One 64-thread block per (row, head).
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
      const float w = __builtin_amdgcn_exp2f(ms - M);
      L += w * part_ml[2 * p + 1];
      const float4* src = reinterpret_cast<const float4*>(part_o + p * kLatent + 8 * lane);
      const float4 a = src[0], c = src[1];
      acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
      acc[4] += w * c.x; acc[5] += w * c.y; acc[6] += w * c.z; acc[7] += w * c.w;
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
  if (lse != nullptr && lane == 0) lse[th] = (L > 0.0f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

AttnPlan plan_attn(int T, int H, int W, int rope_dim) {
  (void)rope_dim;
  AttnPlan p{};
  p.head_groups = (H + kHeads - 1) / kHeads;
  const int units = T * p.head_groups;
  const int max_splits = (W + kKeys - 1) / kKeys;
  int s = (kTargetBlocks + units - 1) / units;
  s = s < 1 ? 1 : (s > max_splits ? max_splits : s);
  const int min_s = (W + kMaxRange - 1) / kMaxRange;
  if (s < min_s) s = min_s;
  int range = (W + s - 1) / s;
  range = (range + kKeys - 1) / kKeys * kKeys;
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
  const int64_t blocks = (int64_t)plan.splits * T * plan.head_groups;
  const float sl2 = sm_scale * kLog2e;
  if (rope_dim == 64)
    hipLaunchKernelGGL(attn_mfma_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q,
                       cache, num_slots, idx, idx_stride, W, H, sl2, plan.range, plan.splits,
                       plan.head_groups, out, lse, part_o, part_ml);
  else
    hipLaunchKernelGGL(attn_mfma_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q,
                       cache, num_slots, idx, idx_stride, W, H, sl2, plan.range, plan.splits,
                       plan.head_groups, out, lse, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(T * H), dim3(64), 0, stream, part_o, part_ml,
                     plan.splits, H, out, lse);
  return hipGetLastError();
}

}  // namespace smla
