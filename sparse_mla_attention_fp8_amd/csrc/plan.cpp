// Launch plan of the attention call (host only): a pure function of the
// sizes, shared by the workspace query and the launch so the two agree.
#include "common.h"

namespace smla {

AttnPlan plan_attn(int T, int H, int W, int rope_dim) {
  (void)rope_dim;
  AttnPlan p{};
  p.head_groups = (H + kHeads - 1) / kHeads;
  const int64_t units = (int64_t)T * p.head_groups;
  const int64_t w = W;
  // a single (row, head group) runs four-wavefront workgroups on 32-key
  // chunks with up to twice the splits, which spreads the row over more CUs
  // (one row, 16 heads: 11.7 against 12.0 us NoPE, 11.5 against 12.1 RoPE;
  // from two units on the eight-wavefront shape is faster)
  const bool single = units == 1;
  const int64_t chunk = single ? kKeys / 2 : kKeys;
  const int64_t max_splits = (w + chunk - 1) / chunk;
  // at most one round of workgroups (one per CU, or two per CU for the
  // four-wavefront shape): a split count that spills a few workgroups into a
  // second round doubles the launch
  int64_t s = units >= kTargetBlocks ? 1 : (single ? 2 * kTargetBlocks : kTargetBlocks) / units;
  s = s > max_splits ? max_splits : s;
  int64_t range;
  if (w <= kMaxRange) {
    // the whole row fits one scan: every split deals the row's valid entries
    // out evenly (range 0), so padding in the buffer costs no split any work
    range = s > 1 ? 0 : w;
  } else {
    // wider buffers: fixed ranges of whole chunks, each at most one scan
    const int64_t min_s = (w + kMaxRange - 1) / kMaxRange;
    if (s < min_s) s = min_s;
    range = (w + s - 1) / s;
    range = (range + kKeys - 1) / kKeys * kKeys;
    s = (w + range - 1) / range;
  }
  p.splits = (int)s;
  p.range = (int)range;
  // more (row, head group) units than one round of eight-wavefront workgroups:
  // four-wavefront workgroups, two per CU, so that one's index load, q split
  // and first gathers overlap the other's chunks
  p.waves = (units > kTargetBlocks || single) ? 4 : 8;
  p.blocks = s * units;
  // with a few splits the last one to finish merges its row: that costs two
  // memory round trips instead of a second launch
  p.fused = (p.waves == 8 && s > 1 && s <= kFusedMaxSplits) ? 1 : 0;
  const size_t partials = (s > 1) ? (size_t)T * (size_t)s * (size_t)H * (kLatent + 2) * sizeof(float) : 0;
  p.arrive_off = partials;     // a multiple of 8
  p.workspace = partials + (p.fused ? (size_t)units * sizeof(unsigned long long) : 0);
  return p;
}

}  // namespace smla
