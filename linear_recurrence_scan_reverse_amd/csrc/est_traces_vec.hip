// Vector-valued eligibility traces over [E, T, D] features.
//
// Each feature column (e, d) follows the scalar trace recurrence of the
// estimator entry (forward-time mirror, gist.science summary of rl-triton,
// "Methodologie" section 1), with the per-step decay gamma*lambda and the
// restart after a terminated or truncated step shared by the D columns of a
// row:
//   e_t[d] = a_t * (t == 0 ? init[d] : e_{t-1}[d]) + x_t[d],
//   a_t = gamma*lambda, or 0 when step t-1 ended an episode (t > 0).
//
// Layout on the GPU: a block of 4 waves owns one row e and 64 consecutive
// feature columns (one per lane, so every load and store of a time step is a
// coalesced 256-byte access).  Time goes in super-tiles of 4 x 16 steps: wave
// w folds its 16 steps with a zero entering value into y_t (per lane) and the
// running decay product A_t (wave-uniform, since a_t does not depend on d), so
// that e_t = A_t * c + y_t once the entering value c is known.  The 4
// chunk maps (A, y_last) meet in LDS; each wave composes those of the waves
// before it to get its c, then stores.  The super-tile's outgoing value is the
// next one's entering value.  All arithmetic is fp64; outputs are rounded
// once (to float32, then to the 16-bit storage format when there is one).
// Block and chunk sizes measured at 1024 x 256 x 64: 4 x 16 (27 us) beat 16 x 8
// (38 us), 8 x 16 (30 us) and 4 x 8 (29 us).
//
// Layouts: env-major x[e][t][d] with flags [E, T] (a row's steps are D apart,
// rows T*D apart), or time-major x[t][e][d] with flags [T, E] (steps E*D apart,
// rows D apart).  Either way one step of a row is D contiguous values.
#include "rlscan_launch.hpp"

namespace rlscan {

struct TraceVecArgs {
  const float* x;        // [E, T, D] or [T, E, D], values in the storage format
  const uint8_t* term;   // [E, T] or [T, E], or NULL
  const uint8_t* trunc;  // [E, T] or [T, E], or NULL
  const float* init;     // [E, D] or NULL
  float* out;            // as x
  int64_t E, T, D;
  double decay;          // gamma * lambda
};

constexpr int kTvChunk = 16;  // steps per wave chunk

template <class S, bool TM>
__global__ void __launch_bounds__(64 * kTvWaves)
trace_vec_kernel(const TraceVecArgs p) {
  __shared__ double s_a[kTvWaves];
  __shared__ double s_b[kTvWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t T = p.T, D = p.D;
  const int64_t ntile_d = (D + 63) / 64;
  const int64_t e = blockIdx.x / ntile_d;
  const int64_t d = (blockIdx.x - e * ntile_d) * 64 + lane;
  const bool col_ok = d < D;
  const int64_t dc = col_ok ? d : D - 1;  // clamped column: loads stay inside the row
  // element (row e, step t, column dc) = base + off: env-major, the row's base
  // and a 32-bit in-row offset t*D + dc (T*D < 2^30 is checked by the C ABI);
  // time-major, the step's wave-uniform base and the column
  const uint32_t D32 = (uint32_t)D, dc32 = (uint32_t)dc;
  auto elem = [&](int64_t t, int64_t& base, uint32_t& off) __attribute__((always_inline)) {
    if constexpr (TM) {
      base = (t * p.E + e) * D;
      off = dc32;
    } else {
      base = e * T * D;
      off = (uint32_t)t * D32 + dc32;
    }
  };
  // flags of (row e, step t) at fb + t * fs
  const int64_t fb = TM ? e : e * T;
  const int64_t fs = TM ? p.E : 1;
  const uint8_t* te = p.term;
  const uint8_t* tr = p.trunc;

  // value entering the super-tile
  double carry = p.init ? (double)load1<S>(p.init, e * D, (uint32_t)dc) : 0.0;
  for (int64_t t0 = 0; t0 < T; t0 += (int64_t)kTvWaves * kTvChunk) {
    const int64_t c0 = t0 + (int64_t)w * kTvChunk;  // this wave's first step
    // ---- loads: the chunk's feature rows, and the done flags of steps c0-1 .. c0+14
    float xv[kTvChunk];
#pragma unroll
    for (int k = 0; k < kTvChunk; ++k) {
      const int64_t t = c0 + k < T ? c0 + k : T - 1;
      int64_t base;
      uint32_t off;
      elem(t, base, off);
      xv[k] = load1<S>(p.x, base, off);
    }
    // lane j < 16 reads the flags of step c0 + j - 1 (the step before each chunk step)
    bool dn = false;
    if (lane < kTvChunk) {
      const int64_t t = c0 + lane - 1;
      if (t >= 0 && t < T) dn = (te && te[fb + t * fs] != 0) || (tr && tr[fb + t * fs] != 0);
    }
    const unsigned long long reset = __builtin_amdgcn_ballot_w64(dn);  // bit k: step c0+k restarts

    // ---- local fold from a zero entering value (repeated below for the outputs,
    // which is cheaper than holding a double per step and lane)
    double A = 1.0, yl = 0.0;
#pragma unroll
    for (int k = 0; k < kTvChunk; ++k) {
      const double a = ((reset >> k) & 1ull) ? 0.0 : p.decay;
      const bool in_row = c0 + k < T;
      A = in_row ? a * A : A;
      yl = in_row ? __builtin_fma(a, yl, (double)xv[k]) : yl;
    }
    s_b[w][lane] = yl;
    if (lane == 0) s_a[w] = A;
    __syncthreads();

    // ---- value entering this wave's chunk: compose the chunks before it
    double c = carry;
    for (int u = 0; u < w; ++u) c = __builtin_fma(s_a[u], c, s_b[u][lane]);
    // the super-tile's outgoing value (all waves compute it; wave-independent)
    double cout = c;
    for (int u = w; u < kTvWaves; ++u) cout = __builtin_fma(s_a[u], cout, s_b[u][lane]);

    // ---- outputs: e_t = A_t * c + y_t, with A_t the decay product up to step t
    double At = 1.0, yk = 0.0;
#pragma unroll
    for (int k = 0; k < kTvChunk; ++k) {
      const double a = ((reset >> k) & 1ull) ? 0.0 : p.decay;
      At = a * At;
      yk = __builtin_fma(a, yk, (double)xv[k]);
      if (col_ok && c0 + k < T) {
        const float v = (float)__builtin_fma(At, c, yk);
        int64_t base;
        uint32_t off;
        elem(c0 + k, base, off);
        if constexpr (__is_same(S, F32S)) __builtin_nontemporal_store(v, at(p.out + base, off));
        else __builtin_nontemporal_store(f32_to_s<S>(v), reinterpret_cast<uint16_t*>(p.out) + base + off);
      }
    }
    carry = cout;
    __syncthreads();  // the LDS maps are rewritten by the next super-tile
  }
}

template <class S>
static const void* trace_vec_fn(bool time_major) {
  return time_major ? reinterpret_cast<const void*>(&trace_vec_kernel<S, true>)
                    : reinterpret_cast<const void*>(&trace_vec_kernel<S, false>);
}

hipError_t launch_traces_vec(int fmt, bool time_major, const float* x, const uint8_t* term, const uint8_t* trunc,
                             const float* init, float* out, int64_t E, int64_t T, int64_t D, double gamma,
                             double lam, hipStream_t s) {
  TraceVecArgs a{x, term, trunc, init, out, E, T, D, gamma * lam};
  const int64_t blocks = E * ((D + 63) / 64);
  // a grid of at most 2^32 - 1 work-items (the C ABI refuses larger shapes first)
  if (!tv_grid_ok(E, D)) return hipErrorInvalidConfiguration;
  const void* fn = fmt == 1   ? trace_vec_fn<Bf16S>(time_major)
                   : fmt == 2 ? trace_vec_fn<F16S>(time_major)
                              : trace_vec_fn<F32S>(time_major);
  void* params[] = {&a};
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(64 * kTvWaves), params, 0, s);
}

}  // namespace rlscan
