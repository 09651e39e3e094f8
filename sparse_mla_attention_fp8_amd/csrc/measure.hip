// Gather-only measurement kernel: the memory traffic of the attention gather
// (the first 528 or 656 bytes of each listed fp8_ds_mla row) with no
// arithmetic on it, so that a benchmark can measure what the memory system
// delivers for a given list of rows -- the ceiling of the attention kernel's
// gather on the same rows.
//
// Mapping: 256 workgroups of 512 threads (one per CU); workgroup w takes a
// contiguous run of the list, copies its slot numbers to LDS, then thread i
// loads the 16-byte segments i, i + 512, ... of the run's rows, eight loads in
// flight per thread.  Entries outside [0, num_slots) are skipped.  The loaded
// words are folded by XOR into one 32-bit value per workgroup and then into
// *sink, so no load can be dropped by the compiler.
#include "common.h"

namespace smla {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBlocks = 256;
constexpr int kProbeMaxRun = 8192;     // list entries per workgroup (LDS)
constexpr int kProbeInFlight = 8;

template <int NSEG>
__global__ __launch_bounds__(kProbeThreads) void gather_rows_kernel(const uint8_t* __restrict__ cache,
                                                                    int64_t num_slots,
                                                                    const int32_t* __restrict__ slots,
                                                                    int64_t n, int run,
                                                                    uint32_t* __restrict__ sink) {
  __shared__ int rows[kProbeMaxRun];
  __shared__ uint32_t fold[kProbeThreads / 64];
  const int64_t first = (int64_t)blockIdx.x * run;
  const int count = (int)max((int64_t)0, min((int64_t)run, n - first));
  for (int i = threadIdx.x; i < count; i += kProbeThreads) {
    const int s = slots[first + i];
    rows[i] = (s >= 0 && (int64_t)s < num_slots) ? s : -1;
  }
  __syncthreads();
  const int nseg = count * NSEG;
  uint32_t acc = 0;
  for (int f0 = threadIdx.x; f0 < nseg; f0 += kProbeThreads * kProbeInFlight) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int f = f0 + u * kProbeThreads;
      v[u] = make_uint4(0, 0, 0, 0);
      if (f < nseg) {
        const int r = f / NSEG, sg = f - r * NSEG;
        const int s = rows[r];
        if (s >= 0) v[u] = *reinterpret_cast<const uint4*>(cache + (int64_t)s * kRowBytes + 16 * sg);
      }
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) fold[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) a ^= fold[w];
    atomicXor(sink, a);
  }
}

}  // namespace

int64_t gather_probe_max_rows() { return (int64_t)kProbeBlocks * kProbeMaxRun; }

hipError_t launch_gather_probe(const uint8_t* cache, int64_t num_slots, int rope_dim, const int32_t* slots,
                               int64_t n, uint32_t* sink, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int run = (int)((n + kProbeBlocks - 1) / kProbeBlocks);
  if (rope_dim == 64) {
    hipLaunchKernelGGL(gather_rows_kernel<kRowBytes / 16>, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                       cache, num_slots, slots, n, run, sink);
  } else {
    hipLaunchKernelGGL(gather_rows_kernel<kNopeRowBytes / 16>, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                       stream, cache, num_slots, slots, n, run, sink);
  }
  return hipGetLastError();
}

}  // namespace smla
