// rlscan_kernel.hpp -- device side of librlscan (gfx950 / CDNA4, wave64).
//
// One kernel template solves every estimator as an affine scan.  The method
// (rl-triton; gist.science summary, "Methodologie" sections 1-2): each step t
// contributes a pair (a_t, b_t) such that x_t = a_t x_{t+1} + b_t (backward)
// or x_t = a_t x_{t-1} + b_t (forward); pairs compose associatively,
//     outer (+) inner = (a_o a_i, b_o + a_o b_i),
// where "inner" is the element nearer the scan's carry.  The pairs are built
// in registers from the raw inputs and never written to memory.
//
// Work decomposition (ours, for 64-wide wavefronts):
//   * A row (one environment) is owned by a team of L lanes (L = 16 or 32:
//     several rows per wave; L = 64: one wave) or of W whole waves.
//   * The row is cut into tiles of SPAN = (lanes in team) * K steps; a lane
//     owns K consecutive steps of a tile (one 16-byte load per input when
//     K = 4).  Lanes are numbered in SCAN order: lane 0 holds the steps nearest
//     the carry (the latest steps for a backward scan), so a backward suffix
//     scan is an ordinary prefix scan over lane index, and a wave still reads
//     one contiguous block of memory.
//   * Per tile: (1) each lane folds its K pairs serially; (2) a log2(L)-step
//     DPP prefix scan over lanes (row_shr 1,2,4,8, row_bcast 15, row_bcast 31);
//     (3) with W > 1 waves, the wave totals go through LDS and every wave
//     applies the totals of the waves nearer the carry; (4) each lane takes
//     its incoming value from its lower neighbour (DPP wave_shr 1) and
//     re-walks its K steps; (5) the epilogue forms the outputs and stores them.
//     Tiles are visited from the carry side, the running value crossing tiles
//     in registers.
//   * Neighbour-step inputs (V_{t+1}, EQ_{t+1} and c_{t+1}, or the previous
//     step's done flag) come from the adjacent lane by DPP; a lane whose
//     neighbour sits in another team/tile reloads that one element (an L1/L2
//     hit: the neighbouring lane's load brought in the line).
// All scan arithmetic is float64; inputs are float32 and each output is
// rounded once.  Each input element is read from HBM once and each output
// written once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlscan {

// ----------------------------------------------------------------- arguments
struct KernelArgs {
  const float* r;       // rewards; signal x (traces, prefix sums); a (generic scan)
  const float* v;       // values V; Q(s_t, a_t) (Retrace); b (generic scan)
  const float* aux;     // log_rhos (V-trace); E_pi Q(s_t, .) (Retrace)
  const float* pi;      // target-policy probability of a_t (Retrace)
  const float* mu;      // behaviour-policy probability of a_t (Retrace)
  const uint8_t* term;  // terminated flags, NULL = none
  const uint8_t* trunc; // truncated flags, NULL = none
  const float* row;     // [E]: bootstrap_value, init or carry; NULL = zeros
  const float* tboot;   // [E,T] successor value at truncated steps; NULL = zeros
  float* out0;          // main output
  float* out1;          // second output (GAE returns, V-trace pg), NULL = none
  int64_t E, T;
  double gamma, lam, rho_bar, c_bar;
};

// Estimator tags (also make the kernel names readable in profiles).
struct DiscountedReturn { static constexpr bool kReverse = true; };
struct TdLambda { static constexpr bool kReverse = true; };
struct Gae { static constexpr bool kReverse = true; };
struct Vtrace { static constexpr bool kReverse = true; };
struct Retrace { static constexpr bool kReverse = true; };
struct EligibilityTrace { static constexpr bool kReverse = false; };
struct EpisodicPrefixSum { static constexpr bool kReverse = false; };
struct LinearScanReverse { static constexpr bool kReverse = true; };
struct LinearScanForward { static constexpr bool kReverse = false; };

template <class Est> struct Traits {
  static constexpr bool kBackwardRl =
      __is_same(Est, DiscountedReturn) || __is_same(Est, TdLambda) || __is_same(Est, Gae) ||
      __is_same(Est, Vtrace) || __is_same(Est, Retrace);
  static constexpr bool kForwardRl = __is_same(Est, EligibilityTrace) || __is_same(Est, EpisodicPrefixSum);
  static constexpr bool kLinear = __is_same(Est, LinearScanReverse) || __is_same(Est, LinearScanForward);
  static constexpr bool kUsesV = __is_same(Est, TdLambda) || __is_same(Est, Gae) ||
                                 __is_same(Est, Vtrace) || __is_same(Est, Retrace) || kLinear;
  static constexpr bool kUsesAux = __is_same(Est, Vtrace) || __is_same(Est, Retrace);
  static constexpr bool kUsesPiMu = __is_same(Est, Retrace);
  static constexpr bool kUsesFlags = kBackwardRl || kForwardRl;
  // Does step t need a value carried by its scan-predecessor (t+1 backward, t-1 forward)?
  static constexpr bool kNeedsNbValue = __is_same(Est, TdLambda) || __is_same(Est, Gae) ||
                                        __is_same(Est, Vtrace) || __is_same(Est, Retrace);
  static constexpr bool kNeedsNbDone = kForwardRl;
};

template <int W> struct BlockShape { static constexpr int kThreads = (W > 4 ? 64 * W : 256); };

// ----------------------------------------------------------------- pair algebra
struct AB {
  double a, b;
};

// outer (+) inner: apply `inner` first, then `outer`.
__device__ __forceinline__ AB compose(const AB& outer, const AB& inner) {
  AB r;
  r.a = outer.a * inner.a;
  r.b = __builtin_fma(outer.a, inner.b, outer.b);
  return r;
}

// ----------------------------------------------------------------- cross-lane moves
// DPP controls (GFX9 encoding): row_shr:n = 0x110+n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143, wave_shr:1 = 0x138.  A lane whose source is outside
// its row / the wave, or whose row is masked off, keeps `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double old, double src) {
  const unsigned long long o = __builtin_bit_cast(unsigned long long, old);
  const unsigned long long s = __builtin_bit_cast(unsigned long long, src);
  const int lo = __builtin_amdgcn_update_dpp((int)(unsigned)o, (int)(unsigned)s, CTRL, ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(unsigned)(o >> 32), (int)(unsigned)(s >> 32), CTRL,
                                             ROW_MASK, 0xf, false);
  return __builtin_bit_cast(double, ((unsigned long long)(unsigned)hi << 32) | (unsigned long long)(unsigned)lo);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ AB dpp_ab(const AB& v) {
  AB r;
  r.a = dpp_f64<CTRL, ROW_MASK>(1.0, v.a);  // identity element (1, 0) where no source
  r.b = dpp_f64<CTRL, ROW_MASK>(0.0, v.b);
  return r;
}

// Inclusive prefix composition over groups of L consecutive lanes (L = 16,
// 32, 64), lower lanes being nearer the carry: lane i ends with
// v_i (+) v_{i-1} (+) ... (+) v_{group start}.
template <int L>
__device__ __forceinline__ AB lane_scan(AB v) {
  static_assert(L == 16 || L == 32 || L == 64, "team width");
  v = compose(v, dpp_ab<0x111, 0xf>(v));  // row_shr:1
  v = compose(v, dpp_ab<0x112, 0xf>(v));  // row_shr:2
  v = compose(v, dpp_ab<0x114, 0xf>(v));  // row_shr:4
  v = compose(v, dpp_ab<0x118, 0xf>(v));  // row_shr:8
  if constexpr (L >= 32) v = compose(v, dpp_ab<0x142, 0xa>(v));  // row_bcast:15 -> rows 1, 3
  if constexpr (L >= 64) v = compose(v, dpp_ab<0x143, 0xc>(v));  // row_bcast:31 -> rows 2, 3
  return v;
}

// Value of lane (i-1) for lane i; lane 0 of the wave gets `old`.
__device__ __forceinline__ double shift_up_f64(double v) { return dpp_f64<0x138, 0xf>(0.0, v); }
__device__ __forceinline__ float shift_up_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x138, 0xf, 0xf, false));
}
__device__ __forceinline__ int shift_up_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x138, 0xf, 0xf, false);
}

// Broadcast of lane (group start + L - 1) to the group.
template <int L>
__device__ __forceinline__ double group_last_f64(double v, int lane) {
  if constexpr (L == 64) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, 63);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), 63);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
  } else {
    return __shfl(v, (lane & ~(L - 1)) + (L - 1), 64);
  }
}

// ----------------------------------------------------------------- loads / stores
template <int K, bool VEC>
__device__ __forceinline__ void load_f32(const float* __restrict__ p, int64_t idx, int nv, float (&o)[K]) {
  if (VEC && nv == K) {
    if constexpr (K == 1) {
      o[0] = p[idx];
    } else if constexpr (K == 2) {
      const float2 t = *reinterpret_cast<const float2*>(p + idx);
      o[0] = t.x; o[1] = t.y;
    } else if constexpr (K == 4) {
      const float4 t = *reinterpret_cast<const float4*>(p + idx);
      o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    } else {
      static_assert(K == 8, "chunk");
      const float4 t0 = *reinterpret_cast<const float4*>(p + idx);
      const float4 t1 = *reinterpret_cast<const float4*>(p + idx + 4);
      o[0] = t0.x; o[1] = t0.y; o[2] = t0.z; o[3] = t0.w;
      o[4] = t1.x; o[5] = t1.y; o[6] = t1.z; o[7] = t1.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m) o[m] = (m < nv) ? p[idx + m] : 0.0f;
  }
}

// Bit m of the result is set iff byte m of the chunk is nonzero (flags).
template <int K, bool VEC>
__device__ __forceinline__ unsigned load_flags(const uint8_t* __restrict__ p, int64_t idx, int nv) {
  unsigned bits = 0;
  if (VEC && nv == K) {
    if constexpr (K == 1) {
      bits = p[idx] != 0;
    } else if constexpr (K == 2) {
      const unsigned w = *reinterpret_cast<const uint16_t*>(p + idx);
      bits = ((w & 0xffu) != 0) | (((w >> 8) != 0) << 1);
    } else if constexpr (K == 4) {
      const unsigned w = *reinterpret_cast<const uint32_t*>(p + idx);
#pragma unroll
      for (int m = 0; m < 4; ++m) bits |= (((w >> (8 * m)) & 0xffu) != 0) << m;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p + idx);
#pragma unroll
      for (int m = 0; m < 4; ++m) bits |= (((w.x >> (8 * m)) & 0xffu) != 0) << m;
#pragma unroll
      for (int m = 0; m < 4; ++m) bits |= (((w.y >> (8 * m)) & 0xffu) != 0) << (m + 4);
    }
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m)
      if (m < nv) bits |= (p[idx + m] != 0) << m;
  }
  return bits;
}

template <int K, bool VEC>
__device__ __forceinline__ void store_f32(float* __restrict__ p, int64_t idx, int nv, const float (&o)[K]) {
  if (VEC && nv == K) {
    if constexpr (K == 1) {
      p[idx] = o[0];
    } else if constexpr (K == 2) {
      *reinterpret_cast<float2*>(p + idx) = make_float2(o[0], o[1]);
    } else if constexpr (K == 4) {
      *reinterpret_cast<float4*>(p + idx) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
      *reinterpret_cast<float4*>(p + idx) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(p + idx + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m)
      if (m < nv) p[idx + m] = o[m];
  }
}

// ----------------------------------------------------------------- the kernel
// Template parameters: estimator tag, team width L (lanes per row when W = 1),
// chunk K (steps per lane per tile), W (waves per row; W > 1 requires L = 64),
// VEC (rows are aligned for K-wide vector accesses and T % K == 0).
template <class Est, int L, int K, int W, bool VEC>
__global__ void __launch_bounds__(BlockShape<W>::kThreads)
scan_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
  constexpr int BLOCK = BlockShape<W>::kThreads;
  constexpr int TEAM_LANES = (W > 1) ? 64 * W : L;
  constexpr int TEAMS = BLOCK / TEAM_LANES;
  constexpr int SPAN = TEAM_LANES * K;
  static_assert(W == 1 || L == 64, "multi-wave teams use full waves");
  static_assert(BLOCK % TEAM_LANES == 0, "block shape");

  __shared__ double s_tot[(W > 1) ? 2 : 1][TEAMS][(W > 1) ? W : 1][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int team = tid / TEAM_LANES;
  const int w = (W > 1) ? ((tid >> 6) % W) : 0;  // wave index inside the team (0 = nearest carry)
  const int g = (W > 1) ? lane : (lane & (L - 1));  // lane index inside the wave's part of the team
  const bool team_first_lane = (g == 0);            // scan-predecessor lives outside this wave

  const int64_t T = p.T;
  const int64_t E = p.E;
  const int64_t ntiles = (T + SPAN - 1) / SPAN;
  const int pos0 = (w * 64 + g) * K;  // scan position (within a tile) of this lane's innermost step

  const double gamma = p.gamma;
  const double lam = p.lam;
  const double gl = gamma * lam;

  for (int64_t row_base = (int64_t)blockIdx.x * TEAMS; row_base < E; row_base += (int64_t)gridDim.x * TEAMS) {
    const int64_t row = row_base + team;
    const bool row_ok = row < E;
    const int64_t off = row_ok ? row * T : 0;

    // Running value entering the next tile from the carry side.
    double C = 0.0;
    float boot_row = 0.0f;
    if constexpr (Tr::kBackwardRl) {
      if (row_ok && p.row) boot_row = p.row[row];
    } else {
      if (row_ok && p.row) C = (double)p.row[row];
    }

    for (int64_t it = 0; it < ntiles; ++it) {
      const int64_t tile = REV ? (ntiles - 1 - it) : it;
      const int64_t tile_start = tile * SPAN;
      // Memory index (within the row) of this lane's lowest-addressed step.
      const int64_t cs = REV ? (tile_start + SPAN - pos0 - K) : (tile_start + pos0);
      int nv = 0;
      if (row_ok) {
        const int64_t rem = T - cs;
        nv = rem <= 0 ? 0 : (rem >= K ? K : (int)rem);
      }
      const int64_t base = off + cs;

      // ---- (a1) raw inputs, memory order m = 0..K-1
      float rr[K], vv[K], xa[K], pp[K], mm[K];
      load_f32<K, VEC>(p.r, base, nv, rr);
      if constexpr (Tr::kUsesV) load_f32<K, VEC>(p.v, base, nv, vv);
      if constexpr (Tr::kUsesAux) load_f32<K, VEC>(p.aux, base, nv, xa);
      if constexpr (Tr::kUsesPiMu) {
        load_f32<K, VEC>(p.pi, base, nv, pp);
        load_f32<K, VEC>(p.mu, base, nv, mm);
      }
      unsigned tbits = 0, rbits = 0;
      if constexpr (Tr::kUsesFlags) {
        if (p.term) tbits = load_flags<K, VEC>(p.term, base, nv);
        if (p.trunc) rbits = load_flags<K, VEC>(p.trunc, base, nv);
      }

      // Per-step quantity handed to the scan-successor: V (TD/GAE/V-trace),
      // EQ and the trace c (Retrace), done flag (forward estimators).
      double cown[K];
      if constexpr (__is_same(Est, Retrace)) {
#pragma unroll
        for (int m = 0; m < K; ++m) {
          const double ratio = (double)pp[m] / (double)mm[m];
          cown[m] = lam * (ratio < 1.0 ? ratio : 1.0);
        }
      }
      // Scan-last step of this lane (outermost): memory m = 0 backward, K-1 forward.
      constexpr int MLAST = REV ? 0 : K - 1;
      float nb_v = 0.0f;   // V_{t+1} / EQ_{t+1} for this lane's innermost step
      double nb_c = 0.0;   // c_{t+1} (Retrace)
      int nb_done = 0;     // done_{t-1} (forward)
      if constexpr (Tr::kNeedsNbValue) {
        const float src = __is_same(Est, Retrace) ? xa[MLAST] : vv[MLAST];
        nb_v = shift_up_f32(src);
        if constexpr (__is_same(Est, Retrace)) nb_c = shift_up_f64(cown[MLAST]);
      }
      if constexpr (Tr::kNeedsNbDone) {
        nb_done = shift_up_i32((int)(((tbits | rbits) >> MLAST) & 1u));
      }
      if (team_first_lane) {
        // Predecessor in scan order is in another wave, team slot or tile: reload it.
        const int64_t tn = REV ? (cs + K) : (cs - 1);  // its memory index within the row
        // needed only if this lane's innermost step exists: m = K-1 backward, m = 0 forward
        const bool inner_ok = REV ? (nv == K) : (nv > 0);
        const bool ok = row_ok && inner_ok && tn >= 0 && tn < T;
        if constexpr (Tr::kNeedsNbValue) {
          nb_v = 0.0f;
          nb_c = 0.0;
          if (ok) {
            if constexpr (__is_same(Est, Retrace)) {
              nb_v = p.aux[off + tn];
              const double ratio = (double)p.pi[off + tn] / (double)p.mu[off + tn];
              nb_c = lam * (ratio < 1.0 ? ratio : 1.0);
            } else {
              nb_v = p.v[off + tn];
            }
          }
        }
        if constexpr (Tr::kNeedsNbDone) {
          nb_done = 0;
          if (ok) nb_done = (p.term && p.term[off + tn]) || (p.trunc && p.trunc[off + tn]);
        }
      }

      // ---- (a2) coefficients, scan order j = 0..K-1 (j = 0 nearest the carry)
      AB e[K];
      double aux0[K];  // per-step extras for the epilogue (V-trace: rho)
      double bootv[K];
      bool contk[K];
      double vnext[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int m = REV ? (K - 1 - j) : j;
        const int64_t t = cs + m;
        const bool valid = m < nv;
        AB c{1.0, 0.0};
        contk[j] = false;
        bootv[j] = 0.0;
        vnext[j] = 0.0;
        aux0[j] = 0.0;
        if constexpr (Tr::kBackwardRl) {
          const bool te = (tbits >> m) & 1u;
          const bool tr = !te && ((rbits >> m) & 1u);
          const bool end = !te && !tr && (t == T - 1);
          const bool cont = !(te || tr || end);
          double bv = 0.0;
          if (valid && tr && p.tboot) bv = (double)p.tboot[off + t];
          if (end) bv = (double)boot_row;
          // value of the successor step's input (scan predecessor): same lane or neighbour
          double nx = 0.0;
          double cn = 0.0;
          if constexpr (Tr::kNeedsNbValue) {
            if (j == 0) {
              nx = (double)nb_v;
              if constexpr (__is_same(Est, Retrace)) cn = nb_c;
            } else {
              const int mp = REV ? m + 1 : m - 1;
              nx = __is_same(Est, Retrace) ? (double)xa[mp] : (double)vv[mp];
              if constexpr (__is_same(Est, Retrace)) cn = cown[mp];
            }
          }
          const double nu = cont ? nx : bv;  // successor value
          const double r = (double)rr[m];
          if constexpr (__is_same(Est, DiscountedReturn)) {
            c.a = cont ? gamma : 0.0;
            c.b = cont ? r : __builtin_fma(gamma, bv, r);
          } else if constexpr (__is_same(Est, TdLambda)) {
            c.a = cont ? gl : 0.0;
            // r + gamma * ((1 - lambda) V_{t+1})  or  r + gamma * boot
            c.b = __builtin_fma(cont ? (gamma - gl) : gamma, nu, r);
          } else if constexpr (__is_same(Est, Gae)) {
            c.a = cont ? gl : 0.0;
            c.b = __builtin_fma(gamma, nu, r) - (double)vv[m];
          } else if constexpr (__is_same(Est, Vtrace)) {
            const double ratio = (double)expf(xa[m]);
            const double rho = ratio < p.rho_bar ? ratio : p.rho_bar;
            const double ct = lam * (ratio < p.c_bar ? ratio : p.c_bar);
            c.a = cont ? gamma * ct : 0.0;
            c.b = rho * (__builtin_fma(gamma, nu, r) - (double)vv[m]);
            aux0[j] = rho;
          } else if constexpr (__is_same(Est, Retrace)) {
            c.a = cont ? gamma * cn : 0.0;
            c.b = __builtin_fma(gamma, nu, r) - (double)vv[m];
          }
          contk[j] = cont;
          bootv[j] = bv;
          vnext[j] = nx;
        } else if constexpr (Tr::kForwardRl) {
          // keep the running value unless the previous step ended an episode
          int prev_done;
          if (j == 0) {
            prev_done = nb_done;
          } else {
            const int mp = m - 1;
            prev_done = (int)(((tbits | rbits) >> mp) & 1u);
          }
          const double keep = (t == 0 || !prev_done) ? 1.0 : 0.0;
          c.a = __is_same(Est, EligibilityTrace) ? gl * keep : keep;
          c.b = (double)rr[m];
        } else {
          c.a = (double)rr[m];
          c.b = (double)vv[m];
        }
        if (!valid) c = AB{1.0, 0.0};
        e[j] = c;
      }

      // ---- (a3) serial fold of this lane's K steps
      AB agg = e[0];
#pragma unroll
      for (int j = 1; j < K; ++j) agg = compose(e[j], agg);

      // ---- (a4) wave scan over lanes
      const AB incl = lane_scan<(W > 1 ? 64 : L)>(agg);

      // ---- (a5) block carry across the waves of a team (LDS)
      double Cw = C;        // value entering this wave's first step
      double C_next = 0.0;  // value leaving the tile
      if constexpr (W > 1) {
        const int buf = (int)(it & 1);
        if (lane == 63) {
          s_tot[buf][team][w][0] = incl.a;
          s_tot[buf][team][w][1] = incl.b;
        }
        __syncthreads();
        double x = C;
#pragma unroll
        for (int u = 0; u < W; ++u) {
          if (u == w) Cw = x;
          x = __builtin_fma(s_tot[buf][team][u][0], x, s_tot[buf][team][u][1]);
        }
        C_next = x;
      }

      // ---- (a6) value entering each lane, then re-walk
      const double y_last = __builtin_fma(incl.a, Cw, incl.b);  // value after this lane's steps
      const double from_below = shift_up_f64(y_last);
      const double x_in = team_first_lane ? Cw : from_below;
      if constexpr (W == 1) C_next = group_last_f64<L>(y_last, lane);

      double xs[K];
      {
        double x = x_in;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          x = __builtin_fma(e[j].a, x, e[j].b);
          xs[j] = x;
        }
      }

      // ---- (a7) epilogue and one store per output
      float o0[K], o1[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int m = REV ? (K - 1 - j) : j;
        double y = xs[j];
        double y1 = 0.0;
        if constexpr (__is_same(Est, Gae)) {
          y1 = y + (double)vv[m];
        } else if constexpr (__is_same(Est, Vtrace)) {
          const double xprev = (j == 0) ? x_in : xs[j - 1];
          const double succ = contk[j] ? (vnext[j] + xprev) : bootv[j];
          y1 = aux0[j] * (__builtin_fma(gamma, succ, (double)rr[m]) - (double)vv[m]);
          y = (double)vv[m] + y;
        } else if constexpr (__is_same(Est, Retrace)) {
          y = (double)vv[m] + y;
        }
        o0[m] = (float)y;
        o1[m] = (float)y1;
      }
      if (nv > 0) {
        store_f32<K, VEC>(p.out0, base, nv, o0);
        if constexpr (__is_same(Est, Gae) || __is_same(Est, Vtrace)) {
          if (p.out1) store_f32<K, VEC>(p.out1, base, nv, o1);
        }
      }
      C = C_next;
    }
  }
}

}  // namespace rlscan
