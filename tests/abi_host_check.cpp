// Host-only driver of the C ABI's argument checks, built with the address
// and undefined-behaviour sanitizers (tests/test_abi_sanitized.py).  The
// launchers are replaced by stubs that count calls, so no GPU is touched:
// every rejected call must return its error code with no launch, every
// accepted one must reach exactly one launcher, and none may trip a sanitizer
// (out-of-bounds access, signed overflow in the size arithmetic, ...).
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../include/sparse_mla.h"
#include "../include/sparse_mla_measure.h"
#include "../sparse_mla_attention_fp8_amd/csrc/common.h"

static int g_launches = 0;
static hipError_t g_result = hipSuccess;

extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "ok" : "stub error"; }

namespace smla {
hipError_t launch_kv_write(const uint16_t*, int64_t, const uint16_t*, int64_t, int, const int64_t*, int64_t,
                           uint8_t*, int64_t, hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_kv_write_bf16(const uint16_t*, int64_t, const uint16_t*, int64_t, int, const int64_t*,
                                int64_t, uint16_t*, int64_t, hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_attn(const uint16_t*, const uint8_t*, int64_t, const int32_t*, int64_t, int, int, int, int,
                       float, uint16_t*, float*, void*, const AttnPlan& plan, hipStream_t) {
  if (plan.blocks < 1 || plan.blocks > 0x7FFFFFFF) { std::printf("bad grid\n"); std::exit(3); }
  ++g_launches; return g_result;
}
hipError_t launch_attn_bf16(const uint16_t*, const uint16_t*, int64_t, const int32_t*, int64_t, int, int, int,
                            int, float, uint16_t*, float*, void*, const AttnPlan& plan, hipStream_t) {
  if (plan.blocks < 1 || plan.blocks > 0x7FFFFFFF) { std::printf("bad grid\n"); std::exit(3); }
  ++g_launches; return g_result;
}
hipError_t launch_gather_upconvert(const uint8_t*, int64_t, int, const int64_t*, int64_t, uint16_t*, int64_t,
                                   hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_split_pages(const uint8_t*, int64_t, int64_t, const int32_t*, int64_t, uint8_t*, int64_t, int,
                              hipStream_t) { ++g_launches; return g_result; }
hipError_t launch_merge(const uint16_t*, const float*, int, int64_t, uint16_t*, float*, hipStream_t) {
  ++g_launches; return g_result;
}
int64_t gather_probe_max_rows() { return 256 * 8192; }
hipError_t launch_gather_probe(const uint8_t*, int64_t, int, const int32_t*, int64_t, uint32_t*, hipStream_t) {
  ++g_launches; return g_result;
}
alignas(256) static unsigned char g_scratch_stub[256];
hipError_t noalloc_scratch(hipStream_t, void** out) { *out = g_scratch_stub; return hipSuccess; }
}  // namespace smla

static int g_fail = 0;
static int g_cases = 0;

// rc must equal want; a launcher is reached iff want == SMLA_OK or SMLA_ELAUNCH
// (or never, for calls that have nothing to do)
static void expect(const char* what, int rc, int want, bool nothing_to_do = false) {
  ++g_cases;
  const bool launched = g_launches == 1;
  const bool want_launch = (want == SMLA_OK || want == SMLA_ELAUNCH) && !nothing_to_do;
  const char* msg = smla_last_error();
  const size_t len = std::strlen(msg);
  bool ok = rc == want && launched == want_launch && len < 512;
  if (want != SMLA_OK && len == 0) ok = false;
  if (!ok) {
    std::printf("FAIL %s: rc %d (want %d), launches %d, msg '%s'\n", what, rc, want, g_launches, msg);
    ++g_fail;
  }
  g_launches = 0;
}

int main() {
  alignas(16) static unsigned char buf[1 << 16];
  void* P = buf;                      // 16-byte aligned stand-in, never dereferenced by the API
  void* Q = buf + 4096;
  void* odd = buf + 8;
  auto* slots = reinterpret_cast<const int64_t*>(buf + 256);
  auto* idx = reinterpret_cast<const int32_t*>(buf + 512);
  hipStream_t s = nullptr;

  // ---- writers
  for (int bf = 0; bf < 2; ++bf) {
    auto kvw = bf ? mla_kv_write_bf16 : mla_kv_write;
    expect("kvw ok", kvw(P, 512, P, 64, 64, slots, 8, Q, 128, s), SMLA_OK);
    expect("kvw nope ok", kvw(P, 576, nullptr, 0, 0, slots, 8, Q, 128, s), SMLA_OK);
    expect("kvw 0 rows", kvw(nullptr, 0, nullptr, 0, 0, nullptr, 0, nullptr, 1, s), SMLA_OK, true);
    expect("kvw rope", kvw(P, 512, P, 64, 32, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw rows<0", kvw(P, 512, P, 64, 64, slots, -1, Q, 128, s), SMLA_EINVAL);
    expect("kvw rows max", kvw(P, 512, P, 64, 64, slots, INT64_MAX, Q, 128, s), SMLA_EUNSUPPORTED);
    expect("kvw slots 0", kvw(P, 512, P, 64, 64, slots, 8, Q, 0, s), SMLA_EINVAL);
    expect("kvw null kv", kvw(nullptr, 512, P, 64, 64, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw null pe", kvw(P, 512, nullptr, 64, 64, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw pe nope", kvw(P, 512, P, 64, 0, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw stride", kvw(P, 511, P, 64, 64, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw stride min", kvw(P, INT64_MIN, P, 64, 64, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw pe stride", kvw(P, 512, P, 63, 64, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw align", kvw(odd, 512, P, 64, 64, slots, 8, Q, 128, s), SMLA_EINVAL);
    expect("kvw slot align", kvw(P, 512, P, 64, 64, slots + 0, 8, odd, 128, s), SMLA_EINVAL);
    g_result = hipErrorInvalidValue;
    expect("kvw launch error", kvw(P, 512, P, 64, 64, slots, 8, Q, 128, s), SMLA_ELAUNCH);
    g_result = hipSuccess;
  }

  // ---- attention (fp8 and bf16 caches share the checks)
  for (int bf = 0; bf < 2; ++bf) {
    auto at = bf ? sparse_mla_attn_bf16 : sparse_mla_attn;
    expect("attn ok", at(P, Q, 4096, idx, 2176, 2176, 256, 16, 0, 0.04f, P, nullptr, nullptr, 0, s), SMLA_OK);
    expect("attn needs ws", at(P, Q, 4096, idx, 2176, 2176, 4, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EWORKSPACE);
    const size_t ws = sparse_mla_attn_workspace_size(4, 16, 2176, 0);
    expect("attn ws ok", at(P, Q, 4096, idx, 2176, 2176, 4, 16, 0, 0.04f, P, nullptr, Q, ws, s), SMLA_OK);
    expect("attn ws short", at(P, Q, 4096, idx, 2176, 2176, 4, 16, 0, 0.04f, P, nullptr, Q, ws - 1, s),
           SMLA_EWORKSPACE);
    expect("attn ws align", at(P, Q, 4096, idx, 2176, 2176, 4, 16, 0, 0.04f, P, nullptr, odd, ws, s),
           SMLA_EINVAL);
    expect("attn T max", at(P, Q, 4096, idx, 2176, 2176, 65535, 128, 64, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_OK);
    expect("attn T over", at(P, Q, 4096, idx, 2176, 2176, 65536, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EUNSUPPORTED);
    expect("attn T int max", at(P, Q, 4096, idx, INT64_MAX, INT_MAX, INT_MAX, 128, 0, 0.04f, P, nullptr, nullptr,
                                0, s), SMLA_EUNSUPPORTED);
    // the widest buffer: ~932k splits of 2,304 entries per row
    expect("attn W max, one row", at(P, Q, 4096, idx, INT_MAX, INT_MAX, 1, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EWORKSPACE);
    expect("attn W max, many rows", at(P, Q, 4096, idx, INT64_MAX, INT_MAX, 65535, 128, 0, 0.04f, P, nullptr, Q,
                                       SIZE_MAX, s), SMLA_EUNSUPPORTED);
    expect("attn H", at(P, Q, 4096, idx, 2176, 2176, 256, 129, 0, 0.04f, P, nullptr, nullptr, 0, s), SMLA_EINVAL);
    expect("attn H0", at(P, Q, 4096, idx, 2176, 2176, 256, 0, 0, 0.04f, P, nullptr, nullptr, 0, s), SMLA_EINVAL);
    expect("attn T0", at(P, Q, 4096, idx, 2176, 2176, 0, 16, 0, 0.04f, P, nullptr, nullptr, 0, s), SMLA_EINVAL);
    expect("attn Tneg", at(P, Q, 4096, idx, 2176, 2176, INT_MIN, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EINVAL);
    expect("attn W0", at(P, Q, 4096, idx, 2176, 0, 256, 16, 0, 0.04f, P, nullptr, nullptr, 0, s), SMLA_EINVAL);
    expect("attn stride<W", at(P, Q, 4096, idx, 2175, 2176, 256, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EINVAL);
    expect("attn slots", at(P, Q, 0, idx, 2176, 2176, 256, 16, 0, 0.04f, P, nullptr, nullptr, 0, s), SMLA_EINVAL);
    expect("attn scale", at(P, Q, 4096, idx, 2176, 2176, 256, 16, 0, 1.0f / 0.0f, P, nullptr, nullptr, 0, s),
           SMLA_EINVAL);
    expect("attn rope", at(P, Q, 4096, idx, 2176, 2176, 256, 16, 65, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EINVAL);
    expect("attn null q", at(nullptr, Q, 4096, idx, 2176, 2176, 256, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_EINVAL);
    expect("attn null out", at(P, Q, 4096, idx, 2176, 2176, 256, 16, 0, 0.04f, nullptr, nullptr, nullptr, 0, s),
           SMLA_EINVAL);
    expect("attn lse align", at(P, Q, 4096, idx, 2176, 2176, 256, 16, 0, 0.04f, P,
                                reinterpret_cast<float*>(buf + 2), nullptr, 0, s), SMLA_EINVAL);
    g_result = hipErrorInvalidValue;
    expect("attn launch error", at(P, Q, 4096, idx, 2176, 2176, 256, 16, 0, 0.04f, P, nullptr, nullptr, 0, s),
           SMLA_ELAUNCH);
    g_result = hipSuccess;
  }
  // the allocation-free call: same checks, the scratch limit instead of a workspace
  expect("noalloc ok", sparse_mla_attn_noalloc(P, Q, 4096, idx, 2176, 2176, 16, 16, 0, 0.04f, P, nullptr, s),
         SMLA_OK);
  expect("noalloc one split", sparse_mla_attn_noalloc(P, Q, 4096, idx, 2176, 2176, 256, 16, 0, 0.04f, P, nullptr,
                                                      s), SMLA_OK);
  expect("noalloc largest narrow plan", sparse_mla_attn_noalloc(P, Q, 4096, idx, 2304, 2304, 1, 128, 64, 0.04f, P,
                                                                nullptr, s), SMLA_OK);
  expect("noalloc too big", sparse_mla_attn_noalloc(P, Q, 4096, idx, 65536, 65536, 256, 16, 0, 0.04f, P, nullptr,
                                                    s), SMLA_EWORKSPACE);
  expect("noalloc W max", sparse_mla_attn_noalloc(P, Q, 4096, idx, INT_MAX, INT_MAX, 65535, 128, 0, 0.04f, P,
                                                  nullptr, s), SMLA_EUNSUPPORTED);
  expect("noalloc null", sparse_mla_attn_noalloc(P, Q, 4096, nullptr, 2176, 2176, 16, 16, 0, 0.04f, P, nullptr,
                                                 s), SMLA_EINVAL);
  expect("noalloc rope", sparse_mla_attn_noalloc(P, Q, 4096, idx, 2176, 2176, 16, 16, 1, 0.04f, P, nullptr, s),
         SMLA_EINVAL);

  // the workspace query never overflows and agrees with the launch's checks
  for (int T : {1, 2, 3, 16, 64, 65, 255, 256, 257, 65535, 65536, INT_MAX, -1})
    for (int W : {1, 63, 64, 2048, 2176, 2304, 2305, 100000, INT_MAX, 0, -5})
      for (int H : {1, 16, 17, 128, 129})
        (void)sparse_mla_attn_workspace_size(T, H, W, ((unsigned)T ^ (unsigned)W) & 1u ? 0 : 64);

  // ---- merge, gather, page re-split
  expect("merge ok", sparse_mla_merge(P, reinterpret_cast<const float*>(Q), 2, 3, 16, Q, nullptr, s), SMLA_OK);
  expect("merge P0", sparse_mla_merge(P, reinterpret_cast<const float*>(Q), 0, 3, 16, Q, nullptr, s), SMLA_EINVAL);
  expect("merge rows", sparse_mla_merge(P, reinterpret_cast<const float*>(Q), 2, INT_MAX, 128, Q, nullptr, s),
         SMLA_EUNSUPPORTED);
  expect("gather ok", mla_gather_upconvert(P, 128, 64, slots, 4, Q, 576, s), SMLA_OK);
  expect("gather 0 rows", mla_gather_upconvert(nullptr, 128, 64, nullptr, 0, nullptr, 0, s), SMLA_OK, true);
  expect("pages 0", mla_split_pages_64(nullptr, 8, 0, nullptr, 0, nullptr, 0, 656, s), SMLA_OK, true);
  expect("gather rows max", mla_gather_upconvert(P, 128, 64, slots, INT64_MAX, Q, 576, s), SMLA_EUNSUPPORTED);
  expect("gather stride", mla_gather_upconvert(P, 128, 0, slots, 4, Q, INT64_MIN, s), SMLA_EINVAL);
  expect("pages ok", mla_split_pages_64(P, 8, 256 * 656, idx, 4, Q, 64 * 656, 656, s), SMLA_OK);
  expect("pages max", mla_split_pages_64(P, 8, 256 * 656, idx, INT64_MAX, Q, 64 * 656, 656, s),
         SMLA_EUNSUPPORTED);
  expect("pages row bytes", mla_split_pages_64(P, 8, INT64_MAX, idx, 4, Q, 64 * 656, INT_MAX - 15, s),
         SMLA_EINVAL);
  expect("pages stride", mla_split_pages_64(P, 8, INT64_MIN, idx, 4, Q, 64 * 656, 656, s), SMLA_EINVAL);
  expect("pages 585-byte rows", mla_split_pages_64(P, 8, 256 * 585, idx, 4, Q, 64 * 585, 585, s), SMLA_OK);
  expect("pages 0-byte rows", mla_split_pages_64(P, 8, 256 * 656, idx, 4, Q, 64 * 656, 0, s), SMLA_EINVAL);

  auto* sink = reinterpret_cast<uint32_t*>(buf + 1024);
  expect("probe ok", smla_gather_rows_probe(P, 4096, 0, idx, 1000, sink, s), SMLA_OK);
  expect("probe 0 rows", smla_gather_rows_probe(nullptr, 4096, 64, nullptr, 0, nullptr, s), SMLA_OK, true);
  expect("probe max", smla_gather_rows_probe(P, 4096, 64, idx, INT64_MAX, sink, s), SMLA_EUNSUPPORTED);
  expect("probe neg", smla_gather_rows_probe(P, 4096, 64, idx, -1, sink, s), SMLA_EINVAL);
  expect("probe rope", smla_gather_rows_probe(P, 4096, 8, idx, 10, sink, s), SMLA_EINVAL);
  expect("probe sink", smla_gather_rows_probe(P, 4096, 0, idx, 10, nullptr, s), SMLA_EINVAL);
  expect("probe align", smla_gather_rows_probe(odd, 4096, 0, idx, 10, sink, s), SMLA_EINVAL);

  std::printf("%d cases, %d failed\n", g_cases, g_fail);
  return g_fail == 0 ? 0 : 1;
}
