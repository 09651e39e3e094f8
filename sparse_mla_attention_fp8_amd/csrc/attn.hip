// Sparse MLA attention over the fp8_ds_mla cache: split-top-k main kernel on
// CDNA4 matrix cores, and the log-sum-exp merge of the splits.
//
// Semantics (sglang PR 47013, Motivation; sglang PR 39288, Root cause (1);
// vLLM PR 55277, Purpose): a query row attends over the valid entries of its
// top-k list (0 <= idx < num_slots).  Padding is never gathered and carries an
// exact zero weight, so NaN-coded bytes in slot 0 cannot reach the output.
//
// Work decomposition.  One 512-thread workgroup (8 wavefronts, two per SIMD)
// per (split, query row, group of 16 heads).  A split owns an equal share of
// the row's valid entries (or, for a buffer wider than one scan, a fixed range
// of it); the workgroup compacts its entries into LDS in buffer order and
// walks them in chunks of 64 keys.  Batches with more (row, head group) units
// than one round of these workgroups run four-wavefront workgroups on 32-key
// chunks instead, two per CU (see Geo):
//
//   gather  Each chunk's 64 rows (656 B, or the 528 B a NoPE reader needs)
//           are copied HBM -> LDS with direct-to-LDS 16-byte loads, once per
//           chunk and shared by all heads, into a ring of 3 stages.  Each
//           wavefront issues a contiguous run of the chunk's 1-KB loads, four
//           per m0 value through the loads' instruction offsets.  Below 4 GiB
//           of cache the loads take a scalar base and a 32-bit per-lane
//           offset (one 24-bit multiply-add per load); larger caches use
//           64-bit per-lane addresses.
//           Entries past the valid count of the last chunk get a copy of the
//           chunk's first valid row (so every LDS operand is finite) and a
//           weight that is exactly zero.
//   QK^T    Wavefront w scores the 16 keys of block w/2 against all 16 heads
//           over latent half w%2 (two 128-dim tiles): S^T = K Q^T on
//           v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales), fed directly with
//           the cached e4m3 codes.  q (bf16) is split into an e4m3 high part
//           and an e4m3 residual after a power-of-two prescale, exact up to
//           e4m3 subnormal flushing, so two fp8 products give the bf16 q.
//           Each tile is scaled by its fp32 tile scale; the RoPE part (bf16)
//           uses v_mfma_f32_16x16x32_bf16.  The two latent halves meet in LDS.
//   softmax Base-2 online softmax, one state per (head, key half): wavefront w
//           owns keys 32(w%2) .. 32(w%2)+31 of every chunk.  The running max is
//           lazy (it moves only when a score passes it by 2^8).
//   P.V     Wavefront w owns latent tile w/2 (128 dims) for its key half:
//           O^T = V^T P^T on v_mfma_f32_16x16x32_fp8_fp8, V^T read from LDS
//           with the 8-bit transpose read, P * scale_tile split into e4m3 high
//           part + residual after a per-head power-of-two normaliser.
//
// Software pipeline: iteration c scores chunk c+1 (QK^T, partial scores to
// LDS) while it runs softmax and P.V on chunk c, whose V^T operands and tile
// scales each P.V wavefront already holds in registers (read one iteration
// earlier).  One workgroup barrier per chunk then both publishes the partial
// scores and releases chunk c's stage, which is refilled at once, so two
// chunks stay in flight while a chunk computes.
//
// The key halves merge through LDS at the end.  With one split the workgroup
// writes the bf16 output and LSE; with several it writes (O unnormalised fp32,
// m, l) partials.  With two or three splits (eight wavefronts) the split of a
// row that finishes last merges them in the same launch: partials go through
// device-coherent stores and loads, and an arrival word per (row, head group)
// in the workspace names the last split.  Otherwise a merge kernel combines
// them (attn_merge_small_kernel up to 16 splits, attn_merge_kernel beyond,
// attn_merge_spread_kernel beyond for calls of at most 64 (row, head) pairs).
// m is kept in log2 units throughout.
#include "common.h"

#include <atomic>
#include <chrono>
#include <random>

namespace smla {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i8v __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Geometry of the fp8 attention kernel for WAVES = 8 (64-key chunks, the two
// key halves of a chunk on different wavefronts) or WAVES = 4 (32-key chunks,
// every P.V wavefront over all keys of its tile; small enough for two
// workgroups per CU).
template <int ROPE, int WAVES>
struct Geo {
  static constexpr int D = kLatent + ROPE;          // q width
  static constexpr int RB = ROPE ? 656 : 528;       // bytes staged per row
  static constexpr int NSEG = RB / 16;              // 16-byte segments per row
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KEYS = 8 * WAVES;            // keys per chunk
  static constexpr int NBLK = KEYS / 16;            // 16-key MFMA blocks per chunk
  static constexpr int STAGE = KEYS * RB;           // bytes per stage
  static constexpr int NST = 3;                     // ring depth: NST - 1 chunks in flight
  static constexpr int NI = (KEYS * NSEG + 63) / 64;   // 1-KB gather instructions per chunk
  // q of a workgroup's 16 heads, rows padded by 16 bytes (see the q staging)
  static constexpr int QBYTES = kHeads * (D * 2 + 16);
  // four-wavefront workgroups stage q in the ring's last stage, which is
  // filled only once q is split, to stay within half of the LDS
  static constexpr bool Q_IN_STAGE = WAVES == 4;
  static_assert(!Q_IN_STAGE || QBYTES <= STAGE, "q must fit a stage");
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14])
constexpr int vm_lgkm0_wait(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }
constexpr int kLgkm0 = vm_lgkm0_wait(63);

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// LDS pointer to byte a of the workgroup's LDS, for reads whose per-lane part
// is fixed and whose stage part is a scalar: the compiler then folds every
// constant offset into the instruction's offset field.
__device__ __forceinline__ const lds_u8* lds_at(uint32_t a) {
  return (const lds_u8*)(uintptr_t)a;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// (native vector and scalar types only: HIP's vector structs cannot be copied
// from an LDS-qualified reference)
template <typename T>
__device__ __forceinline__ T lds_load(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}

// Direct-to-LDS gather loads (16 bytes per lane), issued as inline asm so the
// compiler adds no waits of its own for them: the pipeline below accounts for
// them with explicit vmcnt waits.  Lane l of a load writes LDS at m0 +
// instruction offset + 16 l; the instruction offset is added to the global
// address too, so callers take it off the per-lane address.  m0 is set from
// two scalars (so the LDS address costs no vector instruction) and restored.
//
// Loads 0..3 of a wavefront: m0 = stage + wave_lds, offsets 0, 1024, 2048, 3072.
// Either a scalar 64-bit base plus 32-bit per-lane offsets (caches below
// 4 GiB) or 64-bit per-lane addresses.
__device__ __forceinline__ void dma16x4(const uint8_t* base, uint32_t o0, uint32_t o1, uint32_t o2,
                                        uint32_t o3, uint32_t stage, uint32_t wave_lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %7\n\t"
      "global_load_lds_dwordx4 %4, %7 offset:1024\n\t"
      "global_load_lds_dwordx4 %5, %7 offset:2048\n\t"
      "global_load_lds_dwordx4 %6, %7 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(stage), "s"(wave_lds), "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(base)
      : "memory", "scc");
}
__device__ __forceinline__ void dma16x4(const uint8_t*, const uint8_t* p0, const uint8_t* p1,
                                        const uint8_t* p2, const uint8_t* p3, uint32_t stage,
                                        uint32_t wave_lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off\n\t"
      "global_load_lds_dwordx4 %4, off offset:1024\n\t"
      "global_load_lds_dwordx4 %5, off offset:2048\n\t"
      "global_load_lds_dwordx4 %6, off offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(stage), "s"(wave_lds), "v"(p0), "v"(p1), "v"(p2), "v"(p3)
      : "memory", "scc");
}
// Load 4 + K of a wavefront: m0 = stage + wave_lds + 4096, offset 1024 K.
template <int K>
__device__ __forceinline__ void dma16_hi(const uint8_t* base, uint32_t o, uint32_t stage, uint32_t wave_lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %2\n\t"
      "s_add_u32 m0, m0, 4096\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4 offset:%5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(stage), "s"(wave_lds), "v"(o), "s"(base), "i"(1024 * K)
      : "memory", "scc");
}
template <int K>
__device__ __forceinline__ void dma16_hi(const uint8_t*, const uint8_t* p, uint32_t stage, uint32_t wave_lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_add_u32 m0, %1, %2\n\t"
      "s_add_u32 m0, m0, 4096\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, off offset:%4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(stage), "s"(wave_lds), "v"(p), "i"(1024 * K)
      : "memory", "scc");
}
// q rows: 16 bytes per lane to lds_base + 16 * lane (m0 saved and restored).
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

// The same with a scalar 64-bit base and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16_sbase(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// Load split of a chunk's NI loads over WAVES wavefronts (see the gather
// geometry in attn_mfma_kernel): CNT1 = NI / WAVES each, one more for the last
// R = NI % WAVES.  all_full(j): load j of every wavefront that issues it lies
// wholly inside the chunk's SEGS segments.
template <int NI, int WAVES, int SEGS>
struct GatherGeo {
  static constexpr int R = NI % WAVES;
  static constexpr int CNT1 = NI / WAVES;
  static constexpr int CNT0 = CNT1 + (R ? 1 : 0);
  static constexpr bool all_full(int j) {
    for (int w = 0; w < WAVES; ++w) {
      const int cnt = CNT1 + (w >= WAVES - R ? 1 : 0);
      const int start = w * CNT1 + (w - (WAVES - R) > 0 ? w - (WAVES - R) : 0);
      if (j < cnt && 64 * (start + j + 1) > SEGS) return false;
    }
    return true;
  }
  static_assert(CNT1 >= 4 && CNT0 <= 8, "loads 0..3 of every wavefront share one m0, 4..7 another");
  static_assert(all_full(0) && all_full(1) && all_full(2) && all_full(3), "loads 0..3 must be whole");
};
// The scalar base of the 32-bit gather offsets sits this far below the cache,
// so that offsets stay non-negative after the instruction offset is taken off.
constexpr uint32_t kGatherBias = 4096;

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

// Two floats -> packed bf16 pair (low half = a), round to nearest even, by
// the hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
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

// Max without NaN canonicalisation (operands are never signalling NaNs).
__device__ __forceinline__ float fmax_nc(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float fmax3_nc(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8_nc(const float* v) {
  return fmax_nc(fmax3_nc(fmax3_nc(fmax3_nc(v[0], v[1], v[2]), v[3], v[4]), v[5], v[6]), v[7]);
}

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one head (VALU
// row swaps; no LDS round trip).
__device__ __forceinline__ float max_xg(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax_nc(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nc(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_xg(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS row read by row m of 16-key block bb of a chunk.  Odd blocks are
// rotated by 8 rows: the 16 rows of any block still cover all residues mod 16,
// and the 8 rows a P.V lane group takes from blocks 2s and 2s+1 (rows 4g..4g+3
// of each) now also differ mod 16.  With row strides of 4 or 36 dwords mod 64
// banks, rows that differ mod 16 sit on distinct banks.
__device__ __forceinline__ int key_row(int bb, int m) { return 16 * bb + ((m + 8 * (bb & 1)) & 15); }

__device__ __forceinline__ long pack64(uint32_t lo, uint32_t hi) {
  return (long)(((uint64_t)hi << 32) | lo);
}

// Compacts the valid entries of idx[lo, hi) into list[] in buffer order and
// returns their count.  In round r thread i takes entry lo + THREADS r + i, so
// each wavefront's loads are contiguous and all rounds are issued at once; a
// wavefront ballot per round gives its count, the counts of every (round,
// wavefront) meet in LDS in buffer order, and each lane places its entry at its
// group's base plus the valid lanes below it (mbcnt).  Two barriers in all.
//
// With share_splits > 0 the valid entries are dealt out instead: of the n
// valid entries of [lo, hi), split `split` keeps positions [split * share,
// (split + 1) * share) in buffer order, share = ceil(n / share_splits)
// rounded up to whole KC-key chunks, so the splits of a row get equal work
// wherever its padding sits.
template <int THREADS>
constexpr int scan_rounds() { return (kMaxRange + THREADS - 1) / THREADS; }

template <int THREADS, int KC>
__device__ int compact_valid(const int32_t* __restrict__ idx, int lo, int hi, int64_t num_slots,
                             int* list, int* group_counts /* [scan_rounds * waves] */,
                             int split = 0, int share_splits = 0) {
  constexpr int kScanRounds = scan_rounds<THREADS>();
  constexpr int kWaves = THREADS / 64;
  constexpr int kThreads = THREADS;
  constexpr int kKeys = KC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[kScanRounds];
#pragma unroll
  for (int r = 0; r < kScanRounds; ++r) {
    const int k = lo + kThreads * r + tid;
    v[r] = k < hi ? idx[k] : -1;
  }
  uint64_t m[kScanRounds];
#pragma unroll
  for (int r = 0; r < kScanRounds; ++r) m[r] = __ballot(v[r] >= 0 && (int64_t)v[r] < num_slots);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kScanRounds; ++r) group_counts[r * kWaves + wave] = __popcll(m[r]);
  }
  __syncthreads();
  int base[kScanRounds];
  int total = 0;
#pragma unroll
  for (int r = 0; r < kScanRounds; ++r) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = group_counts[r * kWaves + w];
      if (w == wave) base[r] = total;
      total += c;
    }
  }
  int w0 = 0, w1 = total;   // positions this split keeps
  if (share_splits > 0) {
    const int share = ((total + share_splits - 1) / share_splits + kKeys - 1) / kKeys * kKeys;
    w0 = min(total, split * share);
    w1 = min(total, w0 + share);
  }
#pragma unroll
  for (int r = 0; r < kScanRounds; ++r) {
    if ((m[r] >> lane) & 1ull) {
      const int pos = base[r] + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[r] >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m[r], 0u));
      if (pos >= w0 && pos < w1) list[pos - w0] = v[r];
    }
  }
  __syncthreads();
  return w1 - w0;
}

// Device-coherent 16- and 8-byte accesses (cache policy sc1, device scope)
// through a raw buffer resource: stores write through to the memory side and
// loads miss any copy a cache holds, so a workgroup on one XCD reads what a
// workgroup on another has stored once that one's stores have completed.
constexpr int kBufWord3 = 0x00020000;     // raw buffer, 32-bit data format (gfx9 family)
constexpr int kDeviceScope = 16;          // cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

// Arrival of one split at its (row, head group) word; true for the split that
// arrives last, which then leaves the word zero.  The word holds the call's
// tag (epoch << 8) plus the splits arrived so far; a word with another tag (the
// zero a finished call leaves, or whatever the workspace held) counts as none
// arrived.  Each failed exchange is another split's arrival, so the loop ends
// within `splits` tries.
__device__ __noinline__ bool arrive_last(unsigned long long* word, unsigned long long epoch, int splits) {
  const unsigned long long tag = epoch << 8;
  unsigned long long old = 0;
  int count = 0;
  for (int i = 0; i <= kFusedMaxSplits; ++i) {
    const unsigned long long want = ((old & ~0xFFull) == tag ? old : tag) + 1;
    if (__hip_atomic_compare_exchange_strong(word, &old, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
      count = (int)(want & 0xFF);
      break;
    }
  }
  if (count == splits) __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return count == splits;
}

// Wavefront priority for instruction issue on a SIMD (s_setprio): the index
// scan, the gather issue and the partial-score reads ahead of it run at
// kPrioIssue, the next chunk's operand reads and slot lookups at
// kPrioOperands, the arithmetic at kPrioCompute.  With two workgroups per CU
// the other workgroup's arithmetic then no longer delays a wavefront's
// loads (1,024-row prefill 58.2 -> 55.8 us; decode shapes unchanged).
constexpr int kPrioIssue = 2, kPrioOperands = 1, kPrioCompute = 0;

// SMALL: the cache spans less than 4 GiB, so row byte offsets fit 32 bits.
// WAVES: 8 (one workgroup per CU) or 4 (two per CU), see Geo.
template <int ROPE, bool SMALL, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES == 8 ? 1 : 2) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, int64_t num_slots,
    const int32_t* __restrict__ idx, int64_t idx_stride, int W, int H, float sm_scale_log2,
    int range, int splits, int head_groups, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml, unsigned long long* __restrict__ arrive,
    unsigned long long epoch) {
  using G = Geo<ROPE, WAVES>;
  constexpr int D = G::D, RB = G::RB;
  constexpr int kWaves = WAVES;
  constexpr int kKeys = G::KEYS;
  constexpr int NB = G::NBLK;

  __shared__ __align__(16) uint8_t stages[G::NST * G::STAGE];   // ring of chunk stages
  __shared__ int slot_list[kMaxRange];
  // partial scores xs[chunk & 1][block][dim half][lane] (keys 4g + r of the
  // block); with eight wavefronts this buffer first holds the staged q, until
  // every wavefront has split it
  constexpr int kXsBytes = 2 * NB * 2 * 64 * 16;
  constexpr int kXqBytes = (!G::Q_IN_STAGE && G::QBYTES > kXsBytes) ? G::QBYTES : kXsBytes;
  __shared__ __align__(16) uint8_t xq[kXqBytes];
  float4 (*xs)[NB][2][64] = reinterpret_cast<float4 (*)[NB][2][64]>(xq);
  __shared__ int wave_counts[scan_rounds<G::THREADS>() * kWaves];
  uint8_t* const qstage = G::Q_IN_STAGE ? stages + (G::NST - 1) * G::STAGE : xq;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values are made visibly uniform so that every barrier sits on
  // scalar control flow
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  // QK role: 16 keys (block qb) x 256 dims (half qh, tiles 2qh and 2qh+1) plus
  // RoPE k-step qh.  P.V role: tile pt over keys 32ps..32ps+31 of each chunk;
  // with eight wavefronts each key half (ps) keeps its own online-softmax
  // state, with four every wavefront takes the chunk's 32 keys (ps = 0).
  const int qb = wave >> 1, qh = wave & 1;
  const int pt = WAVES == 8 ? wave >> 1 : wave;
  const int ps = WAVES == 8 ? wave & 1 : 0;
  int b = blockIdx.x;
  const int split = b % splits;
  b /= splits;
  const int hg = b % head_groups;
  // rows last-first: in a causal prefill later rows list more entries, so the
  // longest workgroups are dispatched first and fewer of them trail at the end
  // (rows of a decode batch cost the same either way)
  const int t = (int)(gridDim.x / (unsigned)(splits * head_groups)) - 1 - b / head_groups;

  // ---- q of the group's heads -> LDS (one copy per workgroup, issued before
  // the index scan, into a buffer of its own so that the first gathers need not
  // wait for it), rows padded by 16 bytes so the fragment reads below fall on
  // distinct banks
  const int head = hg * kHeads + n16;
  const bool hvalid = head < H;
  {
    constexpr int kSegs = D / 8;                  // 16-byte segments of a q row
    constexpr int kPitch = kSegs + 1;             // LDS row pitch in segments
    constexpr int kInstr = (kHeads * kPitch + 63) / 64;
    const int nh = min(kHeads, H - hg * kHeads);
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(q + ((int64_t)t * H + hg * kHeads) * D);
    const uint32_t lds_q = lds_addr(qstage);
#pragma unroll
    for (int j = 0; j < (kInstr + kWaves - 1) / kWaves; ++j) {
      const int i = wave + kWaves * j;
      const int f = 64 * i + lane;                // LDS segment
      const int h = f / kPitch, e = f - h * kPitch;
      if (i < kInstr && h < nh && e < kSegs)
        dma16(qsrc + (int64_t)h * D * 2 + 16 * e, lds_q + 1024u * (uint32_t)i);
    }
  }

  // range 0: every split scans the whole row and keeps its share of the valid entries
  const int lo_k = range == 0 ? 0 : split * range;
  const int hi_k = range == 0 ? W : min(W, lo_k + range);
  // (its barriers also publish the staged q: each wavefront's first wait for
  // its index loads covers its earlier q loads)
  __builtin_amdgcn_s_setprio(kPrioIssue);
  const int n = __builtin_amdgcn_readfirstlane(
      compact_valid<G::THREADS, kKeys>(idx + (int64_t)t * idx_stride, lo_k, hi_k, num_slots, slot_list,
                                       wave_counts, split, range == 0 ? splits : 0));
  __builtin_amdgcn_s_setprio(kPrioCompute);
  const int nch = (n + kKeys - 1) / kKeys;

  // q, split below once the first gathers are in flight: latent score = qs *
  // sum_tiles scale_tile * <code, q_hi + q_lo> (log2 units); qhi / qlo are the
  // B operands of v_mfma_scale_f32_16x16x128_f8f6f4, one per tile; qpe the
  // RoPE k-step's bf16 B operand
  i8v qhi[2], qlo[2];
  float qs;
  bf16x8 qpe;

  // ---- gather geometry.  A chunk is NI 1-KB direct-to-LDS loads; lane l of
  // load i takes flat segment 64i + l of the chunk (a 32-key chunk ends halfway
  // through its last load, whose upper 32 lanes load nothing).  Wavefront w
  // issues loads [gstart, gstart + my_cnt): NI / WAVES each, the NI % WAVES
  // left over going one each to the last wavefronts, so that the partial load
  // is a wavefront's extra one.  Load j of a wavefront writes LDS block
  // gstart + j of the stage: m0 = stage + 1024 gstart serves loads 0..3 through
  // the instruction offset 1024 j, and m0 + 4096 the rest (1024 (j - 4)).
  using GG = GatherGeo<G::NI, kWaves, kKeys * G::NSEG>;
  constexpr int CNT0 = GG::CNT0;
  constexpr int CNT1 = GG::CNT1;
  const bool big = wave >= kWaves - GG::R;        // issues CNT0 loads, else CNT1
  const int my_cnt = big ? CNT0 : CNT1;
  const int gstart = wave * CNT1 + max(0, wave - (kWaves - GG::R));
  // row and per-lane address part of each of this lane's segments (fixed for
  // the kernel).  The instruction offset is added to the global address as
  // well, so it is taken off here; with a 32-bit offset from a scalar base the
  // base is moved down by kGatherBias bytes and the offset up, so the offset
  // stays non-negative.
  int seg_row[CNT0], seg_off[CNT0];
  bool seg_ok[CNT0];
#pragma unroll
  for (int j = 0; j < CNT0; ++j) {
    const int f = 64 * (gstart + j) + lane;
    seg_ok[j] = j < my_cnt && f < kKeys * G::NSEG;
    seg_row[j] = seg_ok[j] ? f / G::NSEG : 0;
    seg_off[j] = (seg_ok[j] ? (f - seg_row[j] * G::NSEG) * 16 : 0) - 1024 * (j & 3) +
                 (SMALL ? kGatherBias : 0);
  }
  const uint8_t* const gbase =
      SMALL ? reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(cache) - kGatherBias) : cache;
  // Slots of the next chunk to gather, looked up one iteration ahead so that
  // the loads never wait on an LDS round trip (rows past the valid count take
  // the chunk's first row).
  int slot[CNT0];
  const uint32_t list0 = lds_addr(reinterpret_cast<const uint8_t*>(slot_list));
  auto fetch_slots = [&](int c) {
    const int base = c * kKeys;
    const int nv = min(kKeys, n - base);
    const uint32_t cb = list0 + 4u * (uint32_t)base;      // the chunk's entries (a scalar)
    // (a chunk's positions lie within the list, so the rows past the valid
    // count read stale entries that are replaced below)
#pragma unroll
    for (int j = 0; j < CNT0; ++j) slot[j] = lds_load<int>(lds_at(cb + 4u * (uint32_t)seg_row[j]));
    if (nv < kKeys) {
      const int first = lds_load<int>(lds_at(cb));
#pragma unroll
      for (int j = 0; j < CNT0; ++j) slot[j] = seg_row[j] < nv ? slot[j] : first;
    }
  };
  // this wavefront's first 1-KB block of a stage (a scalar)
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(1024u * (uint32_t)gstart);
  auto addr = [&](int j) {
    if constexpr (SMALL) return __umul24((uint32_t)slot[j], (uint32_t)kRowBytes) + (uint32_t)seg_off[j];
    else return cache + (int64_t)slot[j] * kRowBytes + seg_off[j];
  };
  auto issue = [&](uint32_t stage_in, int c) {
    (void)c;
    const uint32_t stage = __builtin_amdgcn_readfirstlane(stage_in);
    dma16x4(gbase, addr(0), addr(1), addr(2), addr(3), stage, wave_lds);
    // loads 4..CNT0-1: a load that every wavefront issues and that lies wholly
    // inside the chunk needs no per-lane condition (and no exec-mask branch)
    auto hi = [&](auto kc) {
      constexpr int K = decltype(kc)::value, j = 4 + K;
      if constexpr (j < CNT0) {
        if constexpr (j < CNT1 && GG::all_full(j)) {
          dma16_hi<K>(gbase, addr(j), stage, wave_lds);
        } else if constexpr (GG::all_full(j)) {
          if (big) dma16_hi<K>(gbase, addr(j), stage, wave_lds);       // a scalar branch
        } else if (seg_ok[j]) {
          dma16_hi<K>(gbase, addr(j), stage, wave_lds);
        }
      }
    };
    hi(std::integral_constant<int, 0>{});
    hi(std::integral_constant<int, 1>{});
    hi(std::integral_constant<int, 2>{});
    hi(std::integral_constant<int, 3>{});
  };

  // running max (log2 units) of this key half, per head; a finite sentinel
  // until the first valid key, so that exp2(-inf - m_run) is an exact 0
  float m_run = -1e30f;
  float l_run = 0.0f;        // running sum over this lane's keys (4g + r), normalised
  // P normaliser 2^ne_run: oacc and l_run hold O and l times 2^(8 - ne_run),
  // and the exponent offset m_eff = m_run - (8 - ne_run) makes exp2(s - m_eff)
  // come out already normalised
  int ne_run = 8;
  int ne_hi = -126;
  float m_eff = -1e30f;
  f4 oacc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) oacc[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int k8 = n16 >> 1, h8 = n16 & 1;
  // P.V operands of a chunk, read from its stage one iteration ahead: V^T of
  // tile pt for keys 32ps + [0, 32) through the LDS transpose read (within each
  // 16-lane group, source lane 2k+h reads 8 bytes of slot k's row at dims
  // d0 + 8h; lane i then holds dim d0 + i of the group's 8 slots, byte k =
  // slot k), and the tile-pt scales of this lane's 8 keys (4g + r of blocks
  // 2ps and 2ps + 1).
  long va[2][8];
  float sc[2][8];
  // per-lane byte offsets of the P.V operand reads within a stage
  const uint32_t pv_off = key_row(2 * ps + (k8 >> 2), 4 * g + (k8 & 3)) * RB + 128 * pt + 8 * h8;
  const uint32_t sc_off0 = key_row(2 * ps, 4 * g) * RB + kScaleOff + 4 * pt;
  const uint32_t sc_off1 = key_row(2 * ps + 1, 4 * g) * RB + kScaleOff + 4 * pt;
  // stg: the stage's LDS address (wave-uniform)
  auto read_pv = [&](uint32_t stg, long* v, float* s) {
    const lds_u8* vsrc = lds_at(stg + pv_off);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const v2i tv = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vsrc + 16 * cc));
      v[cc] = pack64((uint32_t)tv[0], (uint32_t)tv[1]);
    }
    // slots 4bb..4bb+3 are four consecutive LDS rows
    const lds_u8* srow0 = lds_at(stg + sc_off0);
    const lds_u8* srow1 = lds_at(stg + sc_off1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = lds_load<float>(srow0 + r * RB);
      s[4 + r] = lds_load<float>(srow1 + r * RB);
    }
  };
  // QK^T partial of a chunk: keys 16qb + [0,16), dims half qh.  The products
  // are issued early and combined late, so nothing waits on them in between.
  struct QkLoad { i8v a0, a1; bf16x8 ar; float2 sq[4]; };
  struct QkPart { f4 acc0, acc1, accr; float2 sq[4]; };
  const uint32_t k_off = key_row(qb, n16) * RB + 256 * qh + 32 * g;
  const uint32_t kpe_off = key_row(qb, n16) * RB + kRopeOff + 64 * qh + 16 * g;
  // rows 4g..4g+3 of a block are consecutive LDS rows (key_row adds r to a
  // multiple of 4 below 16), so one base serves all four
  const uint32_t sq_off = key_row(qb, 4 * g) * RB + kScaleOff + 8 * qh;
  auto qk_load = [&](uint32_t stg) {
    QkLoad o;
    const lds_u8* krow = lds_at(stg + k_off);
    const u32x4 p00 = lds_load<u32x4>(krow);
    const u32x4 p01 = lds_load<u32x4>(krow + 16);
    const u32x4 p10 = lds_load<u32x4>(krow + 128);
    const u32x4 p11 = lds_load<u32x4>(krow + 128 + 16);
    if (ROPE) o.ar = lds_load<bf16x8>(lds_at(stg + kpe_off));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x2 v = lds_load<f32x2>(lds_at(stg + sq_off) + r * RB);
      o.sq[r] = make_float2(v.x, v.y);
    }
    o.a0 = i8v{(int)p00.x, (int)p00.y, (int)p00.z, (int)p00.w, (int)p01.x, (int)p01.y, (int)p01.z, (int)p01.w};
    o.a1 = i8v{(int)p10.x, (int)p10.y, (int)p10.z, (int)p10.w, (int)p11.x, (int)p11.y, (int)p11.z, (int)p11.w};
    return o;
  };
  auto qk_mfma = [&](const QkLoad& k) {
    QkPart o;
    const f4 z4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
    o.acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k.a0, qhi[0], z4, 0, 0, 0, 0, 0, 0);
    o.acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k.a1, qhi[1], z4, 0, 0, 0, 0, 0, 0);
    o.accr = z4;
    if (ROPE) o.accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.ar, qpe, z4, 0, 0, 0);
    o.acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k.a0, qlo[0], o.acc0, 0, 0, 0, 0, 0, 0);
    o.acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k.a1, qlo[1], o.acc1, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) o.sq[r] = k.sq[r];
    return o;
  };
  // partial scores (log2 units) of MFMA rows 4g + r, head n16 -> xs[c & 1]
  auto qk_finish = [&](const QkPart& o, int c) {
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lat = o.sq[r].x * o.acc0[r] + o.sq[r].y * o.acc1[r];
      pr[r] = ROPE ? lat * qs + o.accr[r] * sm_scale_log2 : lat * qs;
    }
    xs[c & 1][qb][qh][lane] = make_float4(pr[0], pr[1], pr[2], pr[3]);
  };

  // ---- pipeline: chunk c lives in stage c % NST ----
  // Chunk 0 is issued as soon as the index list is in LDS and q is split while
  // it flies; chunk 1 follows, and the ring's last stage is filled once chunk
  // 0 has landed.  Every compiler-visible global load (the
  // index scan's) has been consumed by then, so the compiler has no reason to
  // emit a vmcnt wait of its own in the loop (it does not count the inline-asm
  // gathers; a wait of its own there would drain the whole pipeline).
  const uint32_t lds0 = lds_addr(stages);
  if (nch > 0) {
    fetch_slots(0);
    __builtin_amdgcn_s_setprio(kPrioIssue);
    issue(lds0, 0);
    __builtin_amdgcn_s_setprio(kPrioCompute);
  }

  // q fragments of head n16: tile 2qh+u, dims 128(2qh+u) + 32g + 8k + [0, 8) -> qraw[4u + k]
  uint4 qraw[8];
  uint4 qpe_raw = make_uint4(0, 0, 0, 0);    // RoPE k-step qh: dims 512 + 32qh + 8g + [0, 8)
  {
    const uint8_t* qlds = qstage + (size_t)n16 * (D * 2 + 16);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qraw[4 * u + k] = *reinterpret_cast<const uint4*>(qlds + 2 * (128 * (2 * qh + u) + 32 * g + 8 * k));
    if (ROPE) qpe_raw = *reinterpret_cast<const uint4*>(qlds + 2 * (kLatent + 32 * qh + 8 * g));
  }

  if (!hvalid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) qraw[i] = make_uint4(0, 0, 0, 0);
    qpe_raw = make_uint4(0, 0, 0, 0);
  }
  // ---- q half -> e4m3 high + residual after a per-(head, half) power of two
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w4[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w4[j] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w4[j] & 0xFFFF0000u)));
    }
  }
  amax = max_xg(amax);
  int qe = 0;   // amax * 2^qe < 256
  if (amax > 0.0f) {
    qe = 134 - (int)((__float_as_uint(amax) >> 23) & 0xFF);
    qe = qe > 126 ? 126 : (qe < -126 ? -126 : qe);
  }
  const float qscale = exp2_pow(qe);
  // latent score = qs * sum_tiles scale_tile * <code, q_hi + q_lo>, already in log2 units
  qs = exp2_pow(-qe) * sm_scale_log2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 w = qraw[4 * u + k];
      const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w4[j] << 16) * qscale;
        x[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u) * qscale;
      }
      uint32_t h0, l0, h1, l1;
      split_e4m3(x[0], x[1], x[2], x[3], h0, l0);
      split_e4m3(x[4], x[5], x[6], x[7], h1, l1);
      qhi[u][2 * k] = (int)h0; qhi[u][2 * k + 1] = (int)h1;
      qlo[u][2 * k] = (int)l0; qlo[u][2 * k + 1] = (int)l1;
    }
  }
  qpe = __builtin_bit_cast(bf16x8, qpe_raw);
  // the other chunks of the ring but the last, which is issued once chunk 0
  // has landed: chunk 0 then shares the memory system with one chunk per
  // workgroup instead of two, and lands sooner (with four wavefronts that
  // stage also holds q until every wavefront has split it)
  constexpr int kFirst = G::NST - 1;
#pragma unroll
  for (int c = 1; c < kFirst; ++c)
    if (c < nch) {
      fetch_slots(c);
      __builtin_amdgcn_s_setprio(kPrioIssue);
      issue(lds0 + (uint32_t)(c * G::STAGE), c);
      __builtin_amdgcn_s_setprio(kPrioCompute);
    }

  // chunk 0: wait for it (the chunks issued after it stay in flight), score
  // it, read its P.V operands
  if (nch > 0) {
    const int ahead = min(kFirst - 1, nch - 1);
    if (ahead <= 0) vm_barrier<0>();
    else if (ahead == 1) { if (big) vm_barrier<CNT0>(); else vm_barrier<CNT1>(); }
    else { if (big) vm_barrier<2 * CNT0>(); else vm_barrier<2 * CNT1>(); }
    // every wavefront has split q by now, so its stage can take its chunk
    if (G::NST - 1 < nch) {
      fetch_slots(G::NST - 1);
      __builtin_amdgcn_s_setprio(kPrioIssue);
      issue(lds0 + (uint32_t)((G::NST - 1) * G::STAGE), G::NST - 1);
      __builtin_amdgcn_s_setprio(kPrioCompute);
    }
    if (G::NST < nch) fetch_slots(G::NST);
    qk_finish(qk_mfma(qk_load(lds0)), 0);
    read_pv(lds0, va[0], sc[0]);
  }
  // One chunk; its P.V operands are in (vc, scc), the next chunk's go to
  // (vn, scn).  The loop runs two chunks per trip with the buffers swapped, so
  // no operand is copied between registers.
  auto step = [&](const int c, const long* vc, const float* scc, long* vn, float* scn) {
    // Chunk c+1 landed (this wave's loads issued after it: chunks c+2 ..
    // c+NST-1 that exist), and after the barrier chunk c's partial scores are
    // visible and nobody reads chunk c's stage any more.
    const int ahead = min(G::NST - 2, nch - 2 - c);
    if (ahead <= 0) vm_barrier<0>();
    else if (ahead == 1) { if (big) vm_barrier<CNT0>(); else vm_barrier<CNT1>(); }
    else { if (big) vm_barrier<2 * CNT0>(); else vm_barrier<2 * CNT1>(); }
    // Chunk c's partial scores are read first, ahead of the gather issue:
    // LDS reads return in order, so the softmax then waits only for these, and
    // the issue runs while they are in flight.
    __builtin_amdgcn_s_setprio(kPrioIssue);
    float4 u[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int h = 0; h < 2; ++h) u[bb][h] = xs[c & 1][2 * ps + bb][h][lane];
    const int cur = c % G::NST;
    if (c + G::NST < nch) issue(lds0 + (uint32_t)(cur * G::STAGE), c + G::NST);
    __builtin_amdgcn_s_setprio(kPrioCompute);

    // ---- next chunk's operands (for the last chunk: stale bytes, results unused) ----
    // (the stage address as an opaque scalar, so that the compiler keeps one
    // base per read instead of one induction variable per address)
    const uint32_t nstg = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(((c + 1) % G::NST) * G::STAGE));
    __builtin_amdgcn_s_setprio(kPrioOperands);
    const QkLoad nk = qk_load(nstg);
    read_pv(nstg, vn, scn);
    if (c + G::NST + 1 < nch) fetch_slots(c + G::NST + 1);
    __builtin_amdgcn_s_setprio(kPrioCompute);

    // ---------------- softmax over keys 32ps + [0,32) of chunk c ----------------
    // An empty key half (last chunk) scores -inf throughout and adds exact zeros.
    const int nv = min(kKeys, n - c * kKeys);
    float sv[8];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sv[4 * bb + 0] = u[bb][0].x + u[bb][1].x;
      sv[4 * bb + 1] = u[bb][0].y + u[bb][1].y;
      sv[4 * bb + 2] = u[bb][0].z + u[bb][1].z;
      sv[4 * bb + 3] = u[bb][0].w + u[bb][1].w;
    }
    if (nv < kKeys) {                   // last chunk: padding rows score -inf
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key_row(2 * ps + (e >> 2), 4 * g + (e & 3)) >= nv) sv[e] = -INFINITY;
    }
    // Lazy running max: it moves only when a score exceeds it by more than
    // 2^8, so p <= 256 and most chunks leave O's scale untouched.  Whether any
    // head moves is a per-lane test and a wave vote; only then does the
    // wavefront reduce across lanes.
    const float lmax = max8_nc(sv);
    const bool moved = __any(lmax > m_run + 8.0f);   // true on the first chunk with a valid key
    float alpha = 1.0f;
    if (moved) {
      const float mloc = max_xg(lmax);
      const float m_new = mloc > m_run + 8.0f ? mloc : m_run;
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 1 unless this head's max moved
      m_run = m_new;
      m_eff = m_run - (float)(8 - ne_run);
    }
    // p * 2^(8 - ne_run) and (P * scale) * 2^(8 - ne_run), the P.V operand
    float pn[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pn[e] = __builtin_amdgcn_exp2f(sv[e] - m_eff);   // -inf -> exactly 0
      y[e] = pn[e] * scc[e];            // padding rows: p = 0, scale finite (a copied row)
    }
    float psum = ((pn[0] + pn[1]) + (pn[2] + pn[3])) + ((pn[4] + pn[5]) + (pn[6] + pn[7]));
    // The normaliser changes only when the max moved or a product outgrows
    // the e4m3 range (448); otherwise it is kept, which needs no cross-lane
    // work.  It is set so that the largest product lands in (64, 128], which
    // leaves room for 3.5x to 7x growth before the next change, and e4m3
    // flushing drops only terms below 2^-16 of the largest one.
    const float ymax = max8_nc(y);
    if (moved || __any(ymax > 448.0f)) {
      const float nm = max_xg(ymax) * exp2_pow(ne_run - 8);   // largest P * scale
      int ne = 0;
      if (nm > 0.0f) {
        const uint32_t bits = __float_as_uint(nm);
        ne = (int)((bits >> 23) & 0xFF) - 127 + ((bits & 0x7FFFFF) ? 1 : 0) + 1;
        ne = ne > 119 ? 119 : (ne < -96 ? -96 : ne);
      }
      // the normaliser stays within 2^96 of the largest one seen, which
      // bounds oacc by 2^(11+9+9+96) < 2^128; with ne >= -96 the normalised p
      // and l stay below 2^(8+8+96+11) per lane.  exp2 flushes results below
      // 2^-126, so a key's p is dropped below 2^(ne - 134): below 2^-23 of the
      // largest one while ne <= 111, i.e. tile maxima under about 2^109.
      ne_hi = ne > ne_hi ? ne : ne_hi;
      ne = ne < ne_hi - 96 ? ne_hi - 96 : ne;
      // a head whose max did not move keeps a normaliser that still fits
      if (alpha == 1.0f && ne <= ne_run) ne = ne_run;
      const float f = exp2_pow(ne_run - ne);   // this chunk: old normaliser -> new
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= f;
      psum *= f;
      const float resc = alpha * f;            // O and l: old max and normaliser -> new
      ne_run = ne;
      m_eff = m_run - (float)(8 - ne);
      if (!__all(resc == 1.0f)) {
        l_run *= resc;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[cc][r] *= resc;
      }
    }
    l_run += psum;
    uint32_t h0, l0, h1, l1;
    split_e4m3(y[0], y[1], y[2], y[3], h0, l0);
    split_e4m3(y[4], y[5], y[6], y[7], h1, l1);
    const long bhi = pack64(h0, h1), blo = pack64(l0, l1);
    // next chunk's QK^T products, then this chunk's P.V, then the next scores
    const QkPart nq = qk_mfma(nk);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      oacc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(vc[cc], bhi, oacc[cc], 0, 0, 0);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      oacc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(vc[cc], blo, oacc[cc], 0, 0, 0);
    if (c + 1 < nch) qk_finish(nq, c + 1);
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, va[0], sc[0], va[1], sc[1]);
    if (c + 1 < nch) step(c + 1, va[1], sc[1], va[0], sc[0]);
  }

  // ---- combine the two key halves (eight wavefronts), then write ------------
  const float post = exp2_pow(ne_run - 8);
  const float l_full = sum_xg(l_run) * post;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[cc][r] *= post;
  // The halves meet in buffers no wavefront can still be reading, so no
  // barrier is needed before they are written: a wavefront still in the last
  // iteration reads only stage nch % NST and the partial scores, so stage
  // (nch + 1) % NST takes O and the index list (read no more) takes (m, l).
  static_assert(WAVES != 8 || (4 * 64 * 128 <= G::STAGE && 256 * sizeof(float2) <= sizeof(slot_list)), "combine buffers");
  float4* mo = reinterpret_cast<float4*>(stages + (uint32_t)(((nch + 1) % G::NST) * G::STAGE));   // [c][pt][lane] (32 KB)
  float2* ml = reinterpret_cast<float2*>(slot_list);                                             // [pt][lane] (m, l)
  const int slot4 = pt * 64 + lane;
  // with four wavefronts every P.V wavefront holds the whole row of its tile:
  // its own state, weight 1, and nothing from another half
  float M = m_run, L = l_full, w0 = 1.0f, w1 = 0.0f;
  // a merge inside this launch needs every wavefront until the row is merged
  const bool fused = WAVES == 8 && arrive != nullptr;
  if constexpr (WAVES == 8) {
    if (ps == 1) {
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        mo[cc * 256 + slot4] = make_float4(oacc[cc][0], oacc[cc][1], oacc[cc][2], oacc[cc][3]);
      ml[slot4] = make_float2(m_run, l_full);
    }
    lds_barrier();
    if (!fused && (ps == 1 || !hvalid)) return;
    if (ps == 0) {
      const float2 o1 = ml[slot4];
      M = fmaxf(m_run, o1.x);
      // (a half without valid keys has l = 0, so its weight does not matter)
      w0 = __builtin_amdgcn_exp2f(m_run - M);
      w1 = __builtin_amdgcn_exp2f(o1.x - M);
      L = w0 * l_full + w1 * o1.y;
    }
  } else {
    if (!hvalid) return;
  }
  auto other_half = [&](int cc) {
    return WAVES == 8 ? mo[cc * 256 + slot4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  // oacc[c][r] (and mo) hold dim 128pt + 16c + 4g + r
  const int dim0 = 128 * pt + 4 * g;
  if (splits == 1) {
    const float il = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t* dst = out + ((int64_t)t * H + head) * kLatent + dim0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float4 u = other_half(cc);
      const float o4[4] = {w0 * oacc[cc][0] + w1 * u.x, w0 * oacc[cc][1] + w1 * u.y,
                           w0 * oacc[cc][2] + w1 * u.z, w0 * oacc[cc][3] + w1 * u.w};
      *reinterpret_cast<uint2*>(dst + 16 * cc) =
          make_uint2(bf16x2_rne(o4[0] * il, o4[1] * il), bf16x2_rne(o4[2] * il, o4[3] * il));
    }
    if (lse != nullptr && pt == 0 && g == 0)
      lse[(int64_t)t * H + head] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  } else if (!fused) {
    const int64_t pidx = ((int64_t)t * splits + split) * H + head;
    float* dst = part_o + pidx * kLatent + dim0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float4 u = other_half(cc);
      *reinterpret_cast<float4*>(dst + 16 * cc) =
          make_float4(w0 * oacc[cc][0] + w1 * u.x, w0 * oacc[cc][1] + w1 * u.y,
                      w0 * oacc[cc][2] + w1 * u.z, w0 * oacc[cc][3] + w1 * u.w);
    }
    if (pt == 0 && g == 0) {
      part_ml[2 * pidx] = M;
      part_ml[2 * pidx + 1] = L;
    }
  } else if constexpr (WAVES == 8) {
    // The row's partials, O [split][head][512] and (m, l) [split][head], through
    // buffer resources based at the row's first entries and device-coherent
    // accesses: every split stores its own, and the split that arrives last
    // reads the others back.
    const int64_t row0 = (int64_t)t * splits * H;
    const uint32_t o_bytes = (uint32_t)(splits * H * kLatent * 4);
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(part_o + row0 * kLatent, o_bytes);
    const __amdgpu_buffer_rsrc_t rm = coherent_rsrc(part_ml + 2 * row0, (uint32_t)(splits * H * 8));
    f4 mine[8];                            // this split's O at (head, dim0 + 16cc + r)
    if (ps == 0 && hvalid) {
      const uint32_t po = (uint32_t)(((split * H + head) * kLatent + dim0) * 4);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const float4 u = other_half(cc);
        mine[cc] = f4{w0 * oacc[cc][0] + w1 * u.x, w0 * oacc[cc][1] + w1 * u.y,
                      w0 * oacc[cc][2] + w1 * u.z, w0 * oacc[cc][3] + w1 * u.w};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, mine[cc]), ro, po + 64 * cc, 0,
                                               kDeviceScope);
      }
      if (pt == 0 && g == 0) {
        const v2i mlv = v2i{(int)__float_as_uint(M), (int)__float_as_uint(L)};
        __builtin_amdgcn_raw_buffer_store_b64(mlv, rm, (uint32_t)((split * H + head) * 8), 0, kDeviceScope);
      }
    }
    // every wavefront's stores have completed before the split arrives
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    int* last = slot_list;                 // the index list is read no more
    if (tid == 0) *last = arrive_last(arrive + (int64_t)t * head_groups + hg, epoch, splits) ? 1 : 0;
    lds_barrier();
    if (*last == 0) return;
    // The last split merges the row where its own values already are: each
    // writer lane combines its 32 outputs (head n16, dims dim0 + 16cc + r)
    // over the splits in split order, its own O from registers and the others'
    // read back, with the merge kernels' inputs and arithmetic (M = max m_s,
    // weights 2^(m_s - M), O = sum w_s O_s / sum w_s l_s), so the bits do not
    // depend on which split is last.
    if (ps == 1 || !hvalid) return;
    float ms[kFusedMaxSplits], ls[kFusedMaxSplits];
    f4 a[kFusedMaxSplits][8];
#pragma unroll
    for (int j = 0; j < kFusedMaxSplits; ++j) {
      const bool load = j < splits && j != split;
      const uint32_t hm = (uint32_t)(j * H + head);
      // Every split's (m, l), this one's included, is read back: a lane's own
      // l can differ in its last bits from the stored one (the P.V wavefronts
      // of the four dim tiles round their exponentials with different
      // normalisers), and using it would make the bits depend on which split
      // happens to finish last.
      const v2i mlv = j < splits ? __builtin_amdgcn_raw_buffer_load_b64(rm, hm * 8, 0, kDeviceScope) : v2i{0, 0};
      ms[j] = j < splits ? __uint_as_float((uint32_t)mlv[0]) : -INFINITY;
      ls[j] = j < splits ? __uint_as_float((uint32_t)mlv[1]) : 0.0f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        a[j][cc] = load ? __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                              ro, (hm * kLatent + dim0 + 16 * cc) * 4, 0, kDeviceScope))
                        : f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float mg = -INFINITY;
#pragma unroll
    for (int j = 0; j < kFusedMaxSplits; ++j) mg = fmaxf(mg, ms[j]);
    const float f0 = __builtin_amdgcn_exp2f(-INFINITY - mg);   // 0, as a merge kernel's first group
    float Lm = 0.0f * f0;
    f4 acc[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) acc[cc] = f4{0.0f, 0.0f, 0.0f, 0.0f} * f0;
#pragma unroll
    for (int j = 0; j < kFusedMaxSplits; ++j) {
      const float w = __builtin_amdgcn_exp2f(ms[j] - mg);   // 0 past the last split
      Lm += w * ls[j];
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const f4 v = j == split ? mine[cc] : a[j][cc];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cc][e] += w * v[e];
      }
    }
    const float inv = (Lm > 0.0f) ? 1.0f / Lm : 0.0f;
    const int64_t th = (int64_t)t * H + head;
    uint16_t* dsto = out + th * kLatent + dim0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      *reinterpret_cast<uint2*>(dsto + 16 * cc) =
          make_uint2(bf16x2_rne(acc[cc][0] * inv, acc[cc][1] * inv), bf16x2_rne(acc[cc][2] * inv, acc[cc][3] * inv));
    if (lse != nullptr && pt == 0 && g == 0) lse[th] = (Lm > 0.0f) ? (mg + __log2f(Lm)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// BF16 KV cache: rows are bf16 [num_slots][512 + ROPE] (1,024 or 1,152
// bytes), the cache form of sglang PR 47013, Speed Tests (its timed writer
// stores 512 bf16 values per row, and its end-to-end runs use a BF16 KV
// cache).  The same pipeline as attn_mfma_kernel, with:
//   * the 512 latent values of each row staged at a 1,040-byte LDS pitch (one
//     idle lane per 65 of the gather lays out a 16-byte pad), so rows start 4
//     banks apart;
//   * with RoPE, the 64 RoPE values of a chunk's keys loaded by the QK^T
//     wavefronts straight into registers (16 bytes per lane: key n16, dims
//     32qh + 8g of the RoPE part), issued right after the chunk's gather and
//     covered by the same waits, two register sets deep; two 66,560-byte
//     stages of whole 1,152-byte rows would not fit beside the index list;
//   * QK^T on v_mfma_f32_16x16x32_bf16 (8 K-steps of 32 dims per 256-dim
//     half), q used as is;
//   * P.V on v_mfma_f32_16x16x32_bf16 with P rounded once to bf16 and V^T
//     read by ds_read_b64_tr_b16: within each 16-lane group, lane 4a+b gets
//     element b of the 8-byte pieces that lanes a, a+4, a+8, a+12 address;
//   * no tile scales and no normaliser (bf16 P covers the whole range).
constexpr int kB16Pitch = 1040;                  // LDS bytes per staged row
constexpr int kB16Stage = kKeys * kB16Pitch;     // 66,560
constexpr int kB16NST = 2;                       // one chunk in flight while one computes
constexpr int kB16Instr = kKeys * (kB16Pitch / 16) / 64;   // 65 x 1-KB loads per chunk
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int ROPE, bool SMALL>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ cache, int64_t num_slots,
    const int32_t* __restrict__ idx, int64_t idx_stride, int W, int H, float sm_scale_log2,
    int range, int splits, int head_groups, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __align__(16) uint8_t stages[kB16NST * kB16Stage];
  __shared__ int slot_list[kMaxRange];
  __shared__ __align__(16) float4 xs[2][4][2][64];
  __shared__ int wave_counts[scan_rounds<kThreads>() * kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int qb = wave >> 1, qh = wave & 1;
  const int pt = wave >> 1, ps = wave & 1;
  int b = blockIdx.x;
  const int split = b % splits;
  b /= splits;
  const int hg = b % head_groups;
  // rows last-first: in a causal prefill later rows list more entries, so the
  // longest workgroups are dispatched first and fewer of them trail at the end
  // (rows of a decode batch cost the same either way)
  const int t = (int)(gridDim.x / (unsigned)(splits * head_groups)) - 1 - b / head_groups;
  const int head = hg * kHeads + n16;
  const bool hvalid = head < H;
  const uint8_t* cache8 = reinterpret_cast<const uint8_t*>(cache);
  constexpr int D = kLatent + ROPE;           // q and cache row width (elements)
  constexpr uint32_t RS = 2u * D;             // cache row bytes

  // ---- q of the group's heads -> LDS at the same padded pitch -------------
  {
    const int nh = min(kHeads, H - hg * kHeads);
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(q + ((int64_t)t * H + hg * kHeads) * D);
    const uint32_t lds_q = lds_addr(stages);
#pragma unroll
    for (int j = 0; j < (17 + kWaves - 1) / kWaves; ++j) {
      const int i = wave + kWaves * j;           // 16 rows x 65 segments = 1,040 -> 17 loads
      const int f = 64 * i + lane;
      const int h = f / 65, e = f - h * 65;
      if (i < 17 && h < nh && e < 64) dma16(qsrc + (int64_t)h * RS + 16 * e, lds_q + 1024u * (uint32_t)i);
    }
  }
  // RoPE k-step qh of head n16: dims 512 + 32qh + 8g + [0, 8), from global memory
  uint4 qpe_raw = make_uint4(0, 0, 0, 0);
  if (ROPE && hvalid)
    qpe_raw = *reinterpret_cast<const uint4*>(q + ((int64_t)t * H + head) * D + kLatent + 32 * qh + 8 * g);
  // range 0: every split scans the whole row and keeps its share of the valid entries
  const int lo_k = range == 0 ? 0 : split * range;
  const int hi_k = range == 0 ? W : min(W, lo_k + range);
  const int n = __builtin_amdgcn_readfirstlane(
      compact_valid<kThreads, kKeys>(idx + (int64_t)t * idx_stride, lo_k, hi_k, num_slots, slot_list,
                                     wave_counts, split, range == 0 ? splits : 0));
  const int nch = (n + kKeys - 1) / kKeys;
  // q fragments (B operand of the K-steps of half qh): dims 256qh + 32s + 8g + [0, 8)
  bf16x8 qf[8];
  {
    const uint8_t* qlds = stages + (size_t)n16 * kB16Pitch;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 v = *reinterpret_cast<const uint4*>(qlds + 2 * (256 * qh + 32 * s + 8 * g));
      if (!hvalid) v = make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const bf16x8 qpe = __builtin_bit_cast(bf16x8, qpe_raw);

  // ---- gather geometry: load i = wave + 8j covers LDS segments 64i + lane;
  // segment f is row f / 65, piece f % 65 (piece 64 is the pad, not loaded)
  constexpr int CNT0 = (kB16Instr + kWaves - 1) / kWaves;   // 9
  constexpr int CNT1 = kB16Instr / kWaves;                  // 8
  const bool big = wave < kB16Instr % kWaves;
  const int my_cnt = big ? CNT0 : CNT1;
  int seg_row[CNT0], seg_off[CNT0];
#pragma unroll
  for (int j = 0; j < CNT0; ++j) {
    const int f = j < my_cnt ? 64 * (wave + kWaves * j) + lane : 64;   // unused loads: a pad piece
    seg_row[j] = f / 65;
    seg_off[j] = (f - seg_row[j] * 65) * 16;                          // 1,024 = the pad
  }
  int slot[CNT0];
  const int pe_row = key_row(qb, n16);         // this lane's key for the RoPE loads
  int pe_slot = 0;
  auto fetch_slots = [&](int c) {
    const int base = c * kKeys;
    const int nv = min(kKeys, n - base);
    if (nv == kKeys) {
#pragma unroll
      for (int j = 0; j < CNT0; ++j) slot[j] = slot_list[base + seg_row[j]];
      if (ROPE) pe_slot = slot_list[base + pe_row];
    } else {
#pragma unroll
      for (int j = 0; j < CNT0; ++j) slot[j] = slot_list[base + (seg_row[j] < nv ? seg_row[j] : 0)];
      if (ROPE) pe_slot = slot_list[base + (pe_row < nv ? pe_row : 0)];
    }
  };
  // the chunk's latent rows -> LDS, then (RoPE) this lane's 16 RoPE bytes ->
  // pe: one more load per wavefront and chunk, behind the chunk's gather
  auto issue = [&](uint32_t stage, uint4& pe) {
#pragma unroll
    for (int j = 0; j < CNT0; ++j) {
      if (j < my_cnt && seg_off[j] < 1024) {
        const uint32_t lds = stage + 1024u * (uint32_t)(wave + kWaves * j);
        if (SMALL) {
          dma16_sbase(cache8, (uint32_t)slot[j] * RS + (uint32_t)seg_off[j], lds);
        } else {
          dma16(cache8 + (int64_t)slot[j] * RS + seg_off[j], lds);
        }
      }
    }
    if (ROPE) {
      const uint8_t* src = cache8 + (SMALL ? (int64_t)((uint32_t)pe_slot * RS) : (int64_t)pe_slot * RS) +
                           2 * (kLatent + 32 * qh + 8 * g);
      pe = *reinterpret_cast<const uint4*>(src);
    }
  };
  uint4 pe_buf[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};   // RoPE rows of chunks c, c+1 (by c & 1)

  float m_run = -1e30f;
  float l_run = 0.0f;
  f4 oacc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) oacc[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // P.V operands of a chunk: V^T of tile pt, dim block cc (16 dims), keys K =
  // 8g + j <-> row key_row(2ps + (j >> 2), 4g + (j & 3)); two transposed reads
  // per block (j = 0..3, then 4..7).  Lane 4a+b of each 16-lane group addresses
  // row (4g + (lane>>2 & 3)) of the block pair at dims d0 + 4(lane & 3).
  const int tr_a = n16 & 3, tr_k = n16 >> 2;
  bf16x8 va[2][8];
  auto read_pv = [&](const uint8_t* stg, bf16x8* v) {
    const uint8_t* r0 = stg + key_row(2 * ps, 4 * g + tr_k) * kB16Pitch + 2 * (128 * pt + 4 * tr_a);
    const uint8_t* r1 = stg + key_row(2 * ps + 1, 4 * g + tr_k) * kB16Pitch + 2 * (128 * pt + 4 * tr_a);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(r0 + 32 * cc));
      const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(r1 + 32 * cc));
      typedef short v8s __attribute__((ext_vector_type(8)));
      const v8s w = v8s{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      v[cc] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // QK^T of a chunk: keys 16qb + [0,16) (row n16 of block qb), dims half qh;
  // K-steps s = 0..7 cover dims 256qh + 32s + [0, 32)
  struct QkLoad { bf16x8 a[8]; };
  auto qk_load = [&](const uint8_t* stg) {
    QkLoad o;
    const uint8_t* krow = stg + key_row(qb, n16) * kB16Pitch + 2 * (256 * qh + 8 * g);
#pragma unroll
    for (int s = 0; s < 8; ++s) o.a[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + 64 * s));
    return o;
  };
  auto qk_mfma = [&](const QkLoad& k, const uint4& pe) {
    const f4 z4 = f4{0.0f, 0.0f, 0.0f, 0.0f};
    f4 e = z4, d = z4;   // two chains of four K-steps (plus the RoPE K-step qh)
#pragma unroll
    for (int s = 0; s < 8; s += 2) {
      e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.a[s], qf[s], e, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.a[s + 1], qf[s + 1], d, 0, 0, 0);
    }
    if (ROPE) e = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pe), qpe, e, 0, 0, 0);
    return e + d;
  };
  auto qk_finish = [&](const f4 acc, int c) {
    xs[c & 1][qb][qh][lane] = make_float4(acc[0] * sm_scale_log2, acc[1] * sm_scale_log2,
                                          acc[2] * sm_scale_log2, acc[3] * sm_scale_log2);
  };

  const uint32_t lds0 = lds_addr(stages);
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();                                   // staged q read by every wavefront
#pragma unroll
  for (int c = 0; c < kB16NST; ++c)
    if (c < nch) {
      fetch_slots(c);
      issue(lds0 + (uint32_t)(c * kB16Stage), pe_buf[c]);
    }
  if (kB16NST < nch) fetch_slots(kB16NST);
  if (nch > 0) {
    // chunk 0 landed: at most chunk 1's loads (its gather, and its RoPE load) outstanding
    constexpr int kPe = ROPE ? 1 : 0;
    if (nch > 1) { if (big) vm_barrier<CNT0 + kPe>(); else vm_barrier<CNT1 + kPe>(); }
    else vm_barrier<0>();
    qk_finish(qk_mfma(qk_load(stages), pe_buf[0]), 0);
    read_pv(stages, va[0]);
  }
  // pc holds chunk c's RoPE loads (reused for chunk c+2), pn chunk c+1's
  auto step = [&](const int c, const bf16x8* vc, bf16x8* vn, uint4& pc, const uint4& pnx) {
    // chunk c+1 landed (nothing issued after it), chunk c's scores visible,
    // chunk c's stage free
    vm_barrier<0>();
    float4 u[2][2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int h = 0; h < 2; ++h) u[bb][h] = xs[c & 1][2 * ps + bb][h][lane];
    const int cur = c % kB16NST;
    if (c + kB16NST < nch) issue(lds0 + (uint32_t)(cur * kB16Stage), pc);
    const uint8_t* nstg = stages + ((c + 1) % kB16NST) * kB16Stage;
    const QkLoad nk = qk_load(nstg);
    read_pv(nstg, vn);
    if (c + kB16NST + 1 < nch) fetch_slots(c + kB16NST + 1);

    const int nv = min(kKeys, n - c * kKeys);
    float sv[8];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      sv[4 * bb + 0] = u[bb][0].x + u[bb][1].x;
      sv[4 * bb + 1] = u[bb][0].y + u[bb][1].y;
      sv[4 * bb + 2] = u[bb][0].z + u[bb][1].z;
      sv[4 * bb + 3] = u[bb][0].w + u[bb][1].w;
    }
    if (nv < kKeys) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key_row(2 * ps + (e >> 2), 4 * g + (e & 3)) >= nv) sv[e] = -INFINITY;
    }
    const float lmax = max8_nc(sv);
    if (__any(lmax > m_run + 8.0f)) {
      const float mloc = max_xg(lmax);
      const float m_new = mloc > m_run + 8.0f ? mloc : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      if (!__all(alpha == 1.0f)) {
        l_run *= alpha;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[cc][r] *= alpha;
      }
    }
    float pn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pn[e] = __builtin_amdgcn_exp2f(sv[e] - m_run);   // -inf -> 0
    l_run += ((pn[0] + pn[1]) + (pn[2] + pn[3])) + ((pn[4] + pn[5]) + (pn[6] + pn[7]));
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)pn[e];
    const f4 nq = qk_mfma(nk, pnx);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) oacc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vc[cc], pb, oacc[cc], 0, 0, 0);
    if (c + 1 < nch) qk_finish(nq, c + 1);
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, va[0], va[1], pe_buf[0], pe_buf[1]);
    if (c + 1 >= nch) break;
    step(c + 1, va[1], va[0], pe_buf[1], pe_buf[0]);
  }

  // ---- combine the two key halves, then write ------------------------------
  const float l_full = sum_xg(l_run);
  lds_barrier();
  float4* mo = reinterpret_cast<float4*>(stages);
  float2* ml = reinterpret_cast<float2*>(stages + 4 * 64 * 128);
  const int slot4 = pt * 64 + lane;
  if (ps == 1) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc)
      mo[cc * 256 + slot4] = make_float4(oacc[cc][0], oacc[cc][1], oacc[cc][2], oacc[cc][3]);
    ml[slot4] = make_float2(m_run, l_full);
  }
  lds_barrier();
  if (ps == 1 || !hvalid) return;
  const float2 o1 = ml[slot4];
  const float M = fmaxf(m_run, o1.x);
  const float w0 = __builtin_amdgcn_exp2f(m_run - M);
  const float w1 = __builtin_amdgcn_exp2f(o1.x - M);
  const float L = w0 * l_full + w1 * o1.y;
  const int dim0 = 128 * pt + 4 * g;
  if (splits == 1) {
    const float il = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t* dst = out + ((int64_t)t * H + head) * kLatent + dim0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float4 u = mo[cc * 256 + slot4];
      const float o4[4] = {w0 * oacc[cc][0] + w1 * u.x, w0 * oacc[cc][1] + w1 * u.y,
                           w0 * oacc[cc][2] + w1 * u.z, w0 * oacc[cc][3] + w1 * u.w};
      const uint32_t lo2 = bf16x2_rne(o4[0] * il, o4[1] * il);
      const uint32_t hi2 = bf16x2_rne(o4[2] * il, o4[3] * il);
      *reinterpret_cast<uint2*>(dst + 16 * cc) = make_uint2(lo2, hi2);
    }
    if (lse != nullptr && pt == 0 && g == 0)
      lse[(int64_t)t * H + head] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  } else {
    const int64_t pidx = ((int64_t)t * splits + split) * H + head;
    float* dst = part_o + pidx * kLatent + dim0;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float4 u = mo[cc * 256 + slot4];
      *reinterpret_cast<float4*>(dst + 16 * cc) =
          make_float4(w0 * oacc[cc][0] + w1 * u.x, w0 * oacc[cc][1] + w1 * u.y,
                      w0 * oacc[cc][2] + w1 * u.z, w0 * oacc[cc][3] + w1 * u.w);
    }
    if (pt == 0 && g == 0) {
      part_ml[2 * pidx] = M;
      part_ml[2 * pidx + 1] = L;
    }
  }
}

// Combines split partials (m in log2 units): M = max m_s, L = sum 2^(m_s - M) l_s,
// O = sum 2^(m_s - M) O_s / L, lse = (M + log2 L) ln 2.  One 512-thread block
// per (row, head): wavefront w sums splits w, w + 8, ... against its own
// running maximum, with eight splits' loads in flight at once; the eight sums
// then meet in LDS, rescaled to the common maximum.  A split without valid
// entries has m = -1e30 and l = 0 (finite partials), so it weighs nothing;
// L = 0 means the row has no valid entry.
constexpr int kMergeWaves = 8;
constexpr int kMergeUnroll = 8;
constexpr int kMergeSpreadMaxRows = 64;   // up to this many (row, head) pairs: attn_merge_spread_kernel

__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_kernel(const float* __restrict__ part_o,
                                                                      const float* __restrict__ part_ml,
                                                                      int splits, int H,
                                                                      uint16_t* __restrict__ out,
                                                                      float* __restrict__ lse) {
  __shared__ float4 po[kMergeWaves][2][64];
  __shared__ float2 pml[kMergeWaves];
  const int th = blockIdx.x;  // t * H + h
  const int t = th / H, hh = th % H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float* ml = part_ml + 2 * ((int64_t)t * splits * H + hh);   // split s at ml[2 * s * H]
  const float* po_base = part_o + ((int64_t)t * splits * H + hh) * kLatent + 8 * lane;  // + s * H * 512
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  float Mw = -INFINITY, L = 0.0f;
  for (int s0 = wave; s0 < splits; s0 += kMergeWaves * kMergeUnroll) {
    float ms[kMergeUnroll], ls[kMergeUnroll];
    float4 a[kMergeUnroll], c[kMergeUnroll];
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) {
      const int s = s0 + kMergeWaves * j;
      const bool in = s < splits;
      ms[j] = in ? ml[2 * (int64_t)s * H] : -INFINITY;
      ls[j] = in ? ml[2 * (int64_t)s * H + 1] : 0.0f;
      const float4* src = reinterpret_cast<const float4*>(po_base + (int64_t)s * H * kLatent);
      a[j] = in ? src[0] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      c[j] = in ? src[1] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float mg = Mw;
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) mg = fmaxf(mg, ms[j]);
    const float f = __builtin_amdgcn_exp2f(Mw - mg);   // 0 on the first group
    L *= f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= f;
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) {
      const float w = __builtin_amdgcn_exp2f(ms[j] - mg);   // 0 for the padding j
      L += w * ls[j];
      acc[0] += w * a[j].x; acc[1] += w * a[j].y; acc[2] += w * a[j].z; acc[3] += w * a[j].w;
      acc[4] += w * c[j].x; acc[5] += w * c[j].y; acc[6] += w * c[j].z; acc[7] += w * c[j].w;
    }
    Mw = mg;
  }
  po[wave][0][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  po[wave][1][lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (lane == 0) pml[wave] = make_float2(Mw, L);
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, pml[w].x);
  float o[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float Lt = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const float2 mlw = pml[w];
    const float f = mlw.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mlw.x - M);   // idle wavefronts
    const float4 x = po[w][0][lane], y = po[w][1][lane];
    o[0] += f * x.x; o[1] += f * x.y; o[2] += f * x.z; o[3] += f * x.w;
    o[4] += f * y.x; o[5] += f * y.y; o[6] += f * y.z; o[7] += f * y.w;
    Lt += f * mlw.y;
  }
  const float inv = (Lt > 0.0f) ? 1.0f / Lt : 0.0f;
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = bf16x2_rne(o[2 * i] * inv, o[2 * i + 1] * inv);
  *reinterpret_cast<uint4*>(out + (int64_t)th * kLatent + 8 * lane) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse != nullptr && lane == 0) lse[th] = (Lt > 0.0f) ? (M + __log2f(Lt)) * kLn2 : -INFINITY;
}


// The same combination for calls with few (row, head) pairs and many splits
// (a single decode row has up to 68): the 512 dims of a pair are spread over
// four blocks of 128 (grid.y), so four times as many CUs pull the partials;
// lane l of a wavefront owns dims 128 y + 2l and + 1.  Arithmetic and split
// order as attn_merge_kernel.
__global__ __launch_bounds__(64 * kMergeWaves) void attn_merge_spread_kernel(const float* __restrict__ part_o,
                                                                             const float* __restrict__ part_ml,
                                                                             int splits, int H,
                                                                             uint16_t* __restrict__ out,
                                                                             float* __restrict__ lse) {
  __shared__ float2 po[kMergeWaves][64];
  __shared__ float2 pml[kMergeWaves];
  const int th = blockIdx.x;  // t * H + h
  const int t = th / H, hh = th % H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d0 = blockIdx.y * 128 + 2 * lane;
  const float* ml = part_ml + 2 * ((int64_t)t * splits * H + hh);   // split s at ml[2 * s * H]
  const float* po_base = part_o + ((int64_t)t * splits * H + hh) * kLatent + d0;  // + s * H * 512
  float acc0 = 0.0f, acc1 = 0.0f;
  float Mw = -INFINITY, L = 0.0f;
  for (int s0 = wave; s0 < splits; s0 += kMergeWaves * kMergeUnroll) {
    float ms[kMergeUnroll], ls[kMergeUnroll];
    float2 a[kMergeUnroll];
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) {
      const int s = s0 + kMergeWaves * j;
      const bool in = s < splits;
      ms[j] = in ? ml[2 * (int64_t)s * H] : -INFINITY;
      ls[j] = in ? ml[2 * (int64_t)s * H + 1] : 0.0f;
      a[j] = in ? *reinterpret_cast<const float2*>(po_base + (int64_t)s * H * kLatent) : make_float2(0.0f, 0.0f);
    }
    float mg = Mw;
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) mg = fmaxf(mg, ms[j]);
    const float f = __builtin_amdgcn_exp2f(Mw - mg);   // 0 on the first group
    L *= f;
    acc0 *= f;
    acc1 *= f;
#pragma unroll
    for (int j = 0; j < kMergeUnroll; ++j) {
      const float w = __builtin_amdgcn_exp2f(ms[j] - mg);   // 0 for the padding j
      L += w * ls[j];
      acc0 += w * a[j].x;
      acc1 += w * a[j].y;
    }
    Mw = mg;
  }
  po[wave][lane] = make_float2(acc0, acc1);
  if (lane == 0) pml[wave] = make_float2(Mw, L);
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, pml[w].x);
  float o0 = 0.0f, o1 = 0.0f, Lt = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    const float2 mlw = pml[w];
    const float f = mlw.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mlw.x - M);   // idle wavefronts
    const float2 x = po[w][lane];
    o0 += f * x.x;
    o1 += f * x.y;
    Lt += f * mlw.y;
  }
  const float inv = (Lt > 0.0f) ? 1.0f / Lt : 0.0f;
  *reinterpret_cast<uint32_t*>(out + (int64_t)th * kLatent + d0) = bf16x2_rne(o0 * inv, o1 * inv);
  if (lse != nullptr && lane == 0 && blockIdx.y == 0) lse[th] = (Lt > 0.0f) ? (M + __log2f(Lt)) * kLn2 : -INFINITY;
}


// The same combination for few splits (at most kMergeSmallMax): one wavefront
// per (row, head), four per 256-thread block; lane l owns dims 8l..8l+7.  The
// splits are taken GROUP at a time with a running maximum, every load of a
// group issued before any is used, so a call costs one memory round trip and
// no LDS: groups of sixteen for nine to sixteen splits, of eight below, where
// the wider group's registers buy nothing.  The eight-wavefront kernel above
// wins only when there are many splits to spread over its wavefronts.
constexpr int kMergeSmallMax = 16;
constexpr int kMergeSmallRows = 4;

template <int GROUP>
__global__ __launch_bounds__(64 * kMergeSmallRows) void attn_merge_small_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits, int H, int rows,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int th = blockIdx.x * kMergeSmallRows + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // t * H + h (wave-uniform)
  if (th >= rows) return;
  const int t = th / H, hh = th % H;
  const float* ml = part_ml + 2 * ((int64_t)t * splits * H + hh);   // split s at ml[2 * s * H]
  const float* po_base = part_o + ((int64_t)t * splits * H + hh) * kLatent + 8 * lane;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  float M = -INFINITY, L = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += GROUP) {
    float ms[GROUP], ls[GROUP];
    float4 a[GROUP], c[GROUP];
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const int s = s0 + j;
      const bool in = s < splits;
      ms[j] = in ? ml[2 * (int64_t)s * H] : -INFINITY;
      ls[j] = in ? ml[2 * (int64_t)s * H + 1] : 0.0f;
      const float4* src = reinterpret_cast<const float4*>(po_base + (int64_t)s * H * kLatent);
      a[j] = in ? src[0] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      c[j] = in ? src[1] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float mg = M;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) mg = fmaxf(mg, ms[j]);
    const float f = __builtin_amdgcn_exp2f(M - mg);   // 0 on the first group
    L *= f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= f;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const float w = __builtin_amdgcn_exp2f(ms[j] - mg);   // 0 for the padding j
      L += w * ls[j];
      acc[0] += w * a[j].x; acc[1] += w * a[j].y; acc[2] += w * a[j].z; acc[3] += w * a[j].w;
      acc[4] += w * c[j].x; acc[5] += w * c[j].y; acc[6] += w * c[j].z; acc[7] += w * c[j].w;
    }
    M = mg;
  }
  const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = bf16x2_rne(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<uint4*>(out + (int64_t)th * kLatent + 8 * lane) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse != nullptr && lane == 0) lse[th] = (L > 0.0f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// Launches the merge that suits the split count.
hipError_t launch_merge(const float* part_o, const float* part_ml, int splits, int T, int H,
                        uint16_t* out, float* lse, hipStream_t stream) {
  const int rows = T * H;
  if (splits <= kMergeSmallMax) {
    if (splits > 8)
      hipLaunchKernelGGL(attn_merge_small_kernel<16>, dim3((rows + kMergeSmallRows - 1) / kMergeSmallRows),
                         dim3(64 * kMergeSmallRows), 0, stream, part_o, part_ml, splits, H, rows, out, lse);
    else
      hipLaunchKernelGGL(attn_merge_small_kernel<8>, dim3((rows + kMergeSmallRows - 1) / kMergeSmallRows),
                         dim3(64 * kMergeSmallRows), 0, stream, part_o, part_ml, splits, H, rows, out, lse);
  } else {
    if (rows <= kMergeSpreadMaxRows)
      hipLaunchKernelGGL(attn_merge_spread_kernel, dim3(rows, kLatent / 128), dim3(64 * kMergeWaves), 0, stream,
                         part_o, part_ml, splits, H, out, lse);
    else
      hipLaunchKernelGGL(attn_merge_kernel, dim3(rows), dim3(64 * kMergeWaves), 0, stream, part_o, part_ml,
                         splits, H, out, lse);
  }
  return hipGetLastError();
}

}  // namespace

// Tags of fused-merge calls: distinct for every call of the process (below
// 2^56), from a random start so that no leftover workspace word matches one.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> counter{[] {
    unsigned long long seed = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    try {
      std::random_device rd;
      seed ^= ((unsigned long long)rd() << 32) | rd();
    } catch (...) {
      // no entropy source: the clock alone still differs between processes
    }
    return seed;
  }()};
  return counter.fetch_add(1, std::memory_order_relaxed) % ((1ull << 56) - 1) + 1;
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
  const int64_t blocks = plan.blocks;
  const float sl2 = sm_scale * kLog2e;
  // row byte offsets fit 32 bits (and slot * 656 fits the 24-bit multiply)
  const bool small = num_slots <= (int64_t)((0xFFFFFFFFull - 2 * kGatherBias) / kRowBytes) &&
                     num_slots < (1 << 24);
  // the fused merge's arrival words, and a tag no earlier call used
  unsigned long long* arrive = nullptr;
  unsigned long long epoch = 0;
  if (plan.fused) {
    arrive = reinterpret_cast<unsigned long long*>(static_cast<uint8_t*>(workspace) + plan.arrive_off);
    epoch = next_epoch();
  }
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(64 * plan.waves), 0, stream, q, cache,
                       num_slots, idx, idx_stride, W, H, sl2, plan.range, plan.splits, plan.head_groups,
                       out, lse, part_o, part_ml, arrive, epoch);
  };
  if (plan.waves == 4) {
    if (rope_dim == 64) {
      if (small) go(attn_mfma_kernel<64, true, 4>); else go(attn_mfma_kernel<64, false, 4>);
    } else {
      if (small) go(attn_mfma_kernel<0, true, 4>); else go(attn_mfma_kernel<0, false, 4>);
    }
  } else {
    if (rope_dim == 64) {
      if (small) go(attn_mfma_kernel<64, true, 8>); else go(attn_mfma_kernel<64, false, 8>);
    } else {
      if (small) go(attn_mfma_kernel<0, true, 8>); else go(attn_mfma_kernel<0, false, 8>);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1 || plan.fused) return e;
  return launch_merge(part_o, part_ml, plan.splits, T, H, out, lse, stream);
}

hipError_t launch_attn_bf16(const uint16_t* q, const uint16_t* cache, int64_t num_slots,
                            const int32_t* idx, int64_t idx_stride, int W, int T, int H,
                            int rope_dim, float sm_scale, uint16_t* out, float* lse, void* workspace,
                            const AttnPlan& plan, hipStream_t stream) {
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (plan.splits > 1) {
    part_o = static_cast<float*>(workspace);
    part_ml = part_o + (size_t)T * plan.splits * H * kLatent;
  }
  const int64_t blocks = plan.blocks;
  const float sl2 = sm_scale * kLog2e;
  // row byte offsets fit 32 bits
  const bool small = num_slots <= (int64_t)(0xFFFFFFFFull / (2 * (kLatent + rope_dim)));
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q, cache, num_slots,
                       idx, idx_stride, W, H, sl2, plan.range, plan.splits, plan.head_groups, out,
                       lse, part_o, part_ml);
  };
  if (rope_dim == 64) {
    if (small) go(attn_bf16_kernel<64, true>); else go(attn_bf16_kernel<64, false>);
  } else {
    if (small) go(attn_bf16_kernel<0, true>); else go(attn_bf16_kernel<0, false>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_merge(part_o, part_ml, plan.splits, T, H, out, lse, stream);
}

}  // namespace smla
