// rlscan_plan.hpp -- how a long row (or a long time-major column) is cut into
// segments, and the grid-size limits the launches keep.  Plain integer
// arithmetic, no HIP calls: the launcher and the kernels use it, and a CPU
// test compiles it with a host C++ compiler and checks every plan of the
// shapes the C ABI accepts.
//
// A segmented launch parks intermediate float64 values (a segment's affine
// map, then the value entering it) in the first elements of the segment's own
// range of the first output.  The invariant this file keeps: every segment
// holds at least kSegMinLen steps, far more than the 8 elements the two
// parked doubles take in a 16-bit format, so nothing parked ever leaves its
// segment or its row.  The segment count is T / len (rounded down) and the
// last segment takes the remainder, between len and 2 len - 1 steps.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#include <hip/hip_runtime.h>
#define RLSCAN_HD __host__ __device__
#else
#define RLSCAN_HD
#endif

namespace rlscan {

// ----------------------------------------------------------------- row-major long rows
constexpr int64_t kSegTile = 256;        // steps per tile (64 lanes x 4)
constexpr int64_t kSegMinT = 16384;      // rows at least this long ...
constexpr int64_t kSegMaxE = 64;         // ... with at most this many rows are segmented
constexpr int64_t kSegMinLen = 4 * kSegTile;
constexpr int64_t kSegWavesPerCu = 32;   // segments aimed for per compute unit

struct SegPlan {
  int64_t len;   // steps per segment (0: scan whole rows)
  int64_t nseg;  // segments per row (1 when len == 0)
};

// First step of segment `seg` and one past its last (the last segment of a
// row takes the remainder).
RLSCAN_HD inline int64_t seg_begin(int64_t seg, int64_t len) { return seg * len; }
RLSCAN_HD inline int64_t seg_end(int64_t seg, int64_t len, int64_t nseg, int64_t T) {
  return seg == nseg - 1 ? T : (seg + 1) * len;
}

// Segments of whole tiles, about kSegWavesPerCu per compute unit over all
// rows, at least kSegMinLen steps each, and at least two per row.
inline SegPlan row_segments(int64_t E, int64_t T, int64_t cus) {
  if (T < kSegMinT || E < 1 || E > kSegMaxE || cus < 1) return SegPlan{0, 1};
  const int64_t target = cus * kSegWavesPerCu;
  const int64_t want = (target + E - 1) / E;
  int64_t len = (T + want - 1) / want;
  len = (len + kSegTile - 1) / kSegTile * kSegTile;
  if (len < kSegMinLen) len = kSegMinLen;
  const int64_t nseg = T / len;
  if (nseg < 2) return SegPlan{0, 1};
  return SegPlan{len, nseg};
}

// ----------------------------------------------------------------- time-major long columns
constexpr int64_t kTmSegStep = 256;  // segment lengths are multiples of this (whole super-tiles)
constexpr int kTmCarrySeg = 16;      // segments one wave of the carry pass composes
constexpr int64_t kTmMaxSeg = 16 * kTmCarrySeg;
constexpr int kTmWaves = 16;         // waves per time-major block (64 environments each)

// With fewer 64-environment column groups than compute units and columns of
// at least 512 steps: about two blocks per compute unit, at most kTmMaxSeg
// segments per column, at least two.
inline SegPlan tm_segments(int64_t E, int64_t T, int64_t cus) {
  const int64_t groups = (E + 63) / 64;
  if (E < 1 || cus < 1 || groups >= cus || T < 2 * kTmSegStep) return SegPlan{0, 1};
  int64_t want = (2 * cus + groups - 1) / groups;
  if (want > kTmMaxSeg) want = kTmMaxSeg;
  int64_t len = (T + want - 1) / want;
  len = (len + kTmSegStep - 1) / kTmSegStep * kTmSegStep;
  const int64_t nseg = T / len;
  if (nseg < 2) return SegPlan{0, 1};
  return SegPlan{len, nseg};
}

// ----------------------------------------------------------------- time-major item form
// Shape part of the item form's routing (tm_item_envs in rlscan_launch.hpp
// adds the pointer alignment and takes the measured rules from there):
// environments per block, 64 or 32, or 0 where the other time-major kernels
// take the call.  A routed shape always has at least one whole 64-step chunk
// and whole blocks, which is what keeps the item kernel's loader and compute
// waves at equal barrier counts, and 64 * E * 4 < 2^31, so chunk resources
// and the out-of-range offset 2^31 stay apart.
//   streams: input streams of the estimator (5: Retrace, 32-environment blocks
//            only); supertile: the steps of one super-tile of tm_kernel;
//   keep_tm: tm_kernel measured faster at exactly one super-tile.
constexpr int64_t kTiChunkSteps = 64;
constexpr int64_t kTiMaxE = (int64_t)1 << 23;
inline int tm_item_block_envs(int64_t E, int64_t T, int64_t cus, int streams, int64_t supertile, bool keep_tm) {
  if (T < kTiChunkSteps || T % kTiChunkSteps != 0 || E < 1 || E >= kTiMaxE || cus < 1) return 0;
  const bool wide = (E + 63) / 64 >= cus;  // a 64-environment column group per CU at least
  if (wide && streams > 3) return 0;
  const int eb = wide ? 64 : 32;
  if (E % eb != 0) return 0;
  if (eb == 64 && T == supertile && keep_tm) return 0;
  const int64_t chunks = T / kTiChunkSteps, blocks = E / eb;
  if (chunks > 16 && 2 * blocks < cus) return 0;
  return eb;
}

// ----------------------------------------------------------------- grid limits
// A launch keeps its grid at or below 2^32 - 1 work-items.  The C ABI refuses
// the shapes past these limits (RLSCAN_ERR_SHAPE) before any HIP call.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
// Time-major: one block of kTmWaves waves per 64-environment column group (a
// segmented launch has fewer groups than compute units, far below this).
constexpr int64_t kTmMaxGroups = kMaxWorkItems / (64 * (int64_t)kTmWaves);
inline bool tm_grid_ok(int64_t E) { return (E + 63) / 64 <= kTmMaxGroups; }
// Vector traces: one block of kTvWaves waves per row and 64 feature columns.
constexpr int kTvWaves = 4;
constexpr int64_t kTvMaxBlocks = kMaxWorkItems / (64 * (int64_t)kTvWaves);
inline bool tv_grid_ok(int64_t E, int64_t D) {
  const int64_t cg = (D + 63) / 64;
  return cg == 0 || E <= kTvMaxBlocks / cg;
}

}  // namespace rlscan
