// rlscan_launch.hpp -- host-side launch of the scan kernel: picks the team
// shape for a row length T and launches one kernel on the caller's stream.
#pragma once

#include "rlscan_kernel.hpp"

namespace rlscan {

struct LaunchShape {
  int L, K, W;  // lanes per team (W == 1), steps per lane per tile, waves per row
};

// Team shape by row length.  Short rows share a wave (16 or 32 lanes each) so
// that every lane still owns a 4-step chunk; rows up to 256 steps are one
// wave; longer rows use 2 or 4 waves whose totals meet in LDS, and rows
// beyond one tile loop over tiles with the carry in registers.
inline LaunchShape pick_shape(int64_t T) {
  if (T <= 16) return {16, 1, 1};
  if (T <= 32) return {16, 2, 1};
  if (T <= 64) return {16, 4, 1};
  if (T <= 128) return {32, 4, 1};
  if (T <= 256) return {64, 4, 1};
  if (T <= 512) return {64, 4, 2};
  return {64, 4, 4};
}

// K-wide vector accesses need every row start aligned: T % K == 0 and every
// array base aligned to its K-element chunk.
inline bool vector_ok(const KernelArgs& a, int K) {
  if (a.T % K != 0) return false;
  const uintptr_t fa = (uintptr_t)(4 * K), ba = (uintptr_t)K;
  const float* fl[] = {a.r, a.v, a.aux, a.pi, a.mu, a.out0, a.out1};
  for (const float* q : fl)
    if (q && ((uintptr_t)q % fa) != 0) return false;
  const uint8_t* bl[] = {a.term, a.trunc};
  for (const uint8_t* q : bl)
    if (q && ((uintptr_t)q % ba) != 0) return false;
  return true;
}

template <class Est, int L, int K, int W, bool VEC>
inline hipError_t launch_one(const KernelArgs& a, hipStream_t s) {
  constexpr int BLOCK = BlockShape<W>::kThreads;
  constexpr int TEAMS = BLOCK / ((W > 1) ? 64 * W : L);
  int64_t blocks = (a.E + TEAMS - 1) / TEAMS;
  const int64_t kMaxBlocks = (int64_t)1 << 30;  // larger E: grid-stride loop in the kernel
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  KernelArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_kernel<Est, L, K, W, VEC>),
                         dim3((unsigned)blocks), dim3(BLOCK), params, 0, s);
}

template <class Est, int L, int K, int W>
inline hipError_t launch_shape(const KernelArgs& a, hipStream_t s) {
  return vector_ok(a, K) ? launch_one<Est, L, K, W, true>(a, s) : launch_one<Est, L, K, W, false>(a, s);
}

template <class Est>
hipError_t launch(const KernelArgs& a, hipStream_t s) {
  const LaunchShape sh = pick_shape(a.T);
  switch (sh.W * 1000 + sh.L * 10 + sh.K) {
    case 1000 + 160 + 1: return launch_shape<Est, 16, 1, 1>(a, s);
    case 1000 + 160 + 2: return launch_shape<Est, 16, 2, 1>(a, s);
    case 1000 + 160 + 4: return launch_shape<Est, 16, 4, 1>(a, s);
    case 1000 + 320 + 4: return launch_shape<Est, 32, 4, 1>(a, s);
    case 1000 + 640 + 4: return launch_shape<Est, 64, 4, 1>(a, s);
    case 2000 + 640 + 4: return launch_shape<Est, 64, 4, 2>(a, s);
    case 4000 + 640 + 4: return launch_shape<Est, 64, 4, 4>(a, s);
    default: return hipErrorInvalidConfiguration;
  }
}

// One translation unit per estimator instantiates launch<Est>.
extern template hipError_t launch<DiscountedReturn>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<TdLambda>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<Gae>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<Vtrace>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<Retrace>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<EligibilityTrace>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<EpisodicPrefixSum>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<LinearScanReverse>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<LinearScanForward>(const KernelArgs&, hipStream_t);

}  // namespace rlscan
