// Host-only check of the segment plans, the time-major item form's shape rule
// and the grid limits in rlscan_plan.hpp
// (compiled with a plain C++ compiler by tests/test_plan.py; no GPU).
//
// For every plan the launcher can make, each segment must hold at least the
// elements its two parked float64 values take (8 in a 16-bit format), the
// segments must tile the row exactly, and the grids must fit 2^32 - 1
// work-items.  `--ceil-rule` checks instead the rule the launcher used before
// (segment count rounded up, so the last segment could hold a single step):
// the same checks must reject it.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "rlscan_plan.hpp"

using namespace rlscan;

static long long g_checked = 0;
static bool g_ceil_rule = false;

#define FAIL(...)                         \
  do {                                    \
    std::printf("FAIL: ");                \
    std::printf(__VA_ARGS__);             \
    std::printf("\n");                    \
    return false;                         \
  } while (0)

// The launcher's row-major plan, or the rounded-up rule it replaced.
static SegPlan plan_rows(int64_t E, int64_t T, int64_t cus) {
  if (!g_ceil_rule) return row_segments(E, T, cus);
  if (T < kSegMinT || E > kSegMaxE) return SegPlan{0, 1};
  const int64_t want = (cus * kSegWavesPerCu + E - 1) / E;
  int64_t len = (T + want - 1) / want;
  len = (len + kSegTile - 1) / kSegTile * kSegTile;
  if (len < kSegMinLen) len = kSegMinLen;
  if (len >= T) return SegPlan{0, 1};
  return SegPlan{len, (T + len - 1) / len};
}

// Segment bounds as the kernels compute them under the rule being checked.
static int64_t end_of(int64_t s, const SegPlan& p, int64_t T) {
  if (!g_ceil_rule) return seg_end(s, p.len, p.nseg, T);
  const int64_t e = (s + 1) * p.len;
  return e < T ? e : T;
}

// parked: elements the two parked doubles take (4 float32, 8 16-bit values)
static bool check_row_plan(int64_t E, int64_t T, int64_t cus) {
  const SegPlan p = plan_rows(E, T, cus);
  ++g_checked;
  if (p.len == 0) {
    if (p.nseg != 1) FAIL("whole rows with nseg %lld", (long long)p.nseg);
    return true;
  }
  if (E < 1 || E > kSegMaxE || T < kSegMinT) FAIL("E=%lld T=%lld should not be segmented", (long long)E, (long long)T);
  if (p.len % kSegTile != 0 || p.len < kSegMinLen) FAIL("E=%lld T=%lld len %lld", (long long)E, (long long)T, (long long)p.len);
  if (p.nseg < 2) FAIL("E=%lld T=%lld nseg %lld", (long long)E, (long long)T, (long long)p.nseg);
  // grid of the per-segment passes: 4 waves (256 work-items) per block
  if ((E * p.nseg + 3) / 4 * 256 > kMaxWorkItems) FAIL("E=%lld T=%lld grid", (long long)E, (long long)T);
  const int64_t parked = 8;
  int64_t prev_end = 0;
  for (int64_t s = 0; s < p.nseg; ++s) {
    const int64_t b = seg_begin(s, p.len), e = end_of(s, p, T);
    if (b != prev_end) FAIL("E=%lld T=%lld segment %lld starts at %lld, not %lld", (long long)E, (long long)T,
                            (long long)s, (long long)b, (long long)prev_end);
    if (e - b < parked)
      FAIL("E=%lld T=%lld len %lld: segment %lld holds %lld steps, fewer than the %lld parked elements",
           (long long)E, (long long)T, (long long)p.len, (long long)s, (long long)(e - b), (long long)parked);
    if (e - b < p.len || e - b >= 2 * p.len)
      FAIL("E=%lld T=%lld segment %lld length %lld outside [len, 2 len)", (long long)E, (long long)T, (long long)s,
           (long long)(e - b));
    prev_end = e;
  }
  if (prev_end != T) FAIL("E=%lld T=%lld segments end at %lld", (long long)E, (long long)T, (long long)prev_end);
  return true;
}

static bool check_tm_plan(int64_t E, int64_t T, int64_t cus) {
  const SegPlan p = tm_segments(E, T, cus);
  ++g_checked;
  const int64_t groups = (E + 63) / 64;
  if (p.len == 0) return p.nseg == 1;
  if (groups >= cus || T < 2 * kTmSegStep) FAIL("tm E=%lld T=%lld should not be segmented", (long long)E, (long long)T);
  if (p.len % kTmSegStep != 0 || p.nseg < 2 || p.nseg > kTmMaxSeg)
    FAIL("tm E=%lld T=%lld len %lld nseg %lld", (long long)E, (long long)T, (long long)p.len, (long long)p.nseg);
  // the carry pass: 16 waves of at most kTmCarrySeg segments
  if ((p.nseg + 15) / 16 > kTmCarrySeg) FAIL("tm E=%lld T=%lld carry", (long long)E, (long long)T);
  if (groups * p.nseg * 64 * kTmWaves > kMaxWorkItems) FAIL("tm E=%lld T=%lld grid", (long long)E, (long long)T);
  int64_t prev_end = 0;
  for (int64_t s = 0; s < p.nseg; ++s) {
    const int64_t b = seg_begin(s, p.len), e = seg_end(s, p.len, p.nseg, T);
    if (b != prev_end || e - b < 8 || e - b < p.len || e - b >= 2 * p.len)
      FAIL("tm E=%lld T=%lld segment %lld [%lld, %lld)", (long long)E, (long long)T, (long long)s, (long long)b,
           (long long)e);
    prev_end = e;
  }
  if (prev_end != T) FAIL("tm E=%lld T=%lld segments end at %lld", (long long)E, (long long)T, (long long)prev_end);
  return true;
}

static bool check_limits() {
  // time-major: one block of kTmWaves waves per 64 environments
  for (int64_t E : {int64_t(1), int64_t(64), kTmMaxGroups * 64 - 1, kTmMaxGroups * 64, kTmMaxGroups * 64 + 1,
                    int64_t(1) << 40}) {
    const bool fits = (E + 63) / 64 * 64 * kTmWaves <= kMaxWorkItems;
    if (tm_grid_ok(E) != fits) FAIL("tm_grid_ok(%lld)", (long long)E);
  }
  for (int64_t D : {int64_t(1), int64_t(64), int64_t(65), int64_t(4096)})
    for (int64_t E : {int64_t(1), kTvMaxBlocks / ((D + 63) / 64), kTvMaxBlocks / ((D + 63) / 64) + 1, int64_t(1) << 40}) {
      const bool fits = E * ((D + 63) / 64) * 64 * kTvWaves <= kMaxWorkItems;
      if (tv_grid_ok(E, D) != fits) FAIL("tv_grid_ok(%lld, %lld)", (long long)E, (long long)D);
    }
  return true;
}

// The time-major item form: a routed shape has whole blocks and at least one
// whole chunk (the kernel's loader and compute waves each meet 1 + T / 64
// barriers, the compute side running its first chunk unconditionally), chunk
// resources below the 2^31 out-of-range offset, five-stream calls in
// 32-environment blocks only, and a grid within 2^32 - 1 work-items.
static bool check_item(int64_t E, int64_t T, int64_t cus, int streams, bool keep_tm) {
  ++g_checked;
  const int64_t supertile = streams >= 3 ? 128 : 256;
  const int eb = tm_item_block_envs(E, T, cus, streams, supertile, keep_tm);
  if (eb == 0) return true;
  if (eb != 32 && eb != 64) FAIL("item E=%lld T=%lld: %d environments per block", (long long)E, (long long)T, eb);
  if (T < kTiChunkSteps || T % kTiChunkSteps != 0)
    FAIL("item E=%lld T=%lld: not whole chunks", (long long)E, (long long)T);
  if (E < 1 || E % eb != 0) FAIL("item E=%lld T=%lld: not whole blocks of %d", (long long)E, (long long)T, eb);
  if (streams > 3 && eb != 32) FAIL("item E=%lld: five streams in blocks of %d", (long long)E, eb);
  if (kTiChunkSteps * E * 4 >= ((int64_t)1 << 31)) FAIL("item E=%lld: a chunk resource reaches 2^31", (long long)E);
  if (E / eb * 64 * (eb / 8 + eb / 16) > kMaxWorkItems) FAIL("item E=%lld: grid too large", (long long)E);
  if (T / kTiChunkSteps > 0x7fffffff) FAIL("item T=%lld: chunk count", (long long)T);
  return true;
}

int main(int argc, char** argv) {
  g_ceil_rule = argc > 1 && std::strcmp(argv[1], "--ceil-rule") == 0;
  const int64_t cus_list[] = {256, 304, 80, 8, 1};
  // every row length from 16000 to 40000 at 256 compute units, for 1..65 rows
  for (int64_t E = 1; E <= 65; ++E)
    for (int64_t T = 16000; T <= 40000; ++T)
      if (!check_row_plan(E, T, 256)) return 1;
  // T = k * len + r around segment multiples, up to the longest row, other CU counts
  for (int64_t cus : cus_list)
    for (int64_t E : {int64_t(1), int64_t(2), int64_t(3), int64_t(17), int64_t(63), int64_t(64)}) {
      for (int64_t k = 16; k < (int64_t(1) << 30) / 1024; k = k * 5 / 4 + 1)
        for (int64_t len : {int64_t(1024), int64_t(1280), int64_t(4096), int64_t(65536)})
          for (int64_t r = -8; r <= 8; ++r) {
            const int64_t T = k * len + r;
            if (T >= 1 && T < (int64_t(1) << 30) && !check_row_plan(E, T, cus)) return 1;
          }
      if (!check_row_plan(E, (int64_t(1) << 30) - 1, cus)) return 1;
    }
  if (g_ceil_rule) {
    std::printf("OK %lld plans\n", g_checked);
    return 0;
  }
  // time-major: few column groups and long columns
  for (int64_t cus : cus_list)
    for (int64_t E : {int64_t(2), int64_t(63), int64_t(64), int64_t(65), int64_t(130), int64_t(4000), int64_t(16383)})
      for (int64_t T = 1; T < 70000; T += (T < 3000 ? 1 : 97))
        if (!check_tm_plan(E, T, cus)) return 1;
  // time-major item form: environment counts around the block sizes and the
  // limit, step counts around chunk multiples, every stream count
  for (int64_t cus : cus_list)
    for (int64_t E : {int64_t(1), int64_t(31), int64_t(32), int64_t(33), int64_t(64), int64_t(96), int64_t(4096),
                      int64_t(8192), int64_t(16320), int64_t(16384), int64_t(16416), int64_t(32768),
                      (int64_t(1) << 23) - 64, (int64_t(1) << 23) - 32, int64_t(1) << 23, (int64_t(1) << 23) + 64})
      for (int64_t T : {int64_t(0), int64_t(1), int64_t(63), int64_t(64), int64_t(65), int64_t(128), int64_t(256),
                        int64_t(320), int64_t(1024), int64_t(1088), int64_t(2048), int64_t(2112), int64_t(1) << 20,
                        (int64_t(1) << 30) - 64})
        for (int streams : {1, 2, 3, 5})
          for (bool keep : {false, true})
            if (!check_item(E, T, cus, streams, keep)) return 1;
  if (!check_limits()) return 1;
  std::printf("OK %lld plans\n", g_checked);
  return 0;
}
