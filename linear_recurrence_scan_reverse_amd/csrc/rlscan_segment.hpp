// rlscan_segment.hpp -- long rows with few rows: every row is cut into segments
// of whole 256-step tiles that separate waves scan in parallel.
//
// A row scanned by one wave (or one 4-wave team) walks its tiles one after
// another; with few rows most of the GPU then idles.  Because the pair
// operator is associative, a row can instead be split (gist.science summary
// of rl-triton, "Methodologie" section 1: the O(log T) scan rests on exactly
// this): each segment's steps compose into one affine map x_in -> A x_in + B,
// the maps are scanned per row to give every segment the value entering it,
// and each segment is then scanned again from that value.  Three launches on
// the caller's stream:
//   1. aggregate: one wave per (row, segment) composes the segment's pairs
//      into (A, B);
//   2. carry: one wave per row scans the segment maps in scan order (the same
//      64-lane scan, over segments) and gives each segment its entering value;
//   3. apply: one wave per (row, segment) rescans the segment from that value
//      and writes the outputs.
// Inputs are read twice, outputs written once.  Between the passes, the
// segment's (A, B) and then its entering value live in the first 16 bytes of
// the segment's own range of the first output, which pass 3 overwrites;
// nothing else is allocated.
#pragma once

#include "rlscan_kernel.hpp"
#include "rlscan_plan.hpp"

namespace rlscan {

// A double kept in the first 8 bytes at element `idx` of an output array in
// storage format S (bit copies, element-aligned stores).
template <class S>
__device__ __forceinline__ void put_f64(float* base, int64_t idx, double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  if constexpr (__is_same(S, F32S)) {
    base[idx] = __builtin_bit_cast(float, (unsigned)u);
    base[idx + 1] = __builtin_bit_cast(float, (unsigned)(u >> 32));
  } else {
    uint16_t* b = reinterpret_cast<uint16_t*>(base) + idx;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (uint16_t)(u >> (16 * i));
  }
}
template <class S>
__device__ __forceinline__ double get_f64(const float* base, int64_t idx) {
  unsigned long long u = 0;
  if constexpr (__is_same(S, F32S)) {
    u = (unsigned long long)__builtin_bit_cast(unsigned, base[idx]) |
        ((unsigned long long)__builtin_bit_cast(unsigned, base[idx + 1]) << 32);
  } else {
    const uint16_t* b = reinterpret_cast<const uint16_t*>(base) + idx;
#pragma unroll
    for (int i = 0; i < 4; ++i) u |= (unsigned long long)b[i] << (16 * i);
  }
  return __builtin_bit_cast(double, u);
}
// elements of format S that hold one double
template <class S>
constexpr int f64_elems() { return __is_same(S, F32S) ? 2 : 4; }

// Passes 1 (AGG) and 3 (apply).  One wave per (row, segment); segments are
// seg_len steps (a multiple of 256), and the last one of a row takes the
// remainder (seg_len to 2 seg_len - 1 steps), so the parked pair always lies
// inside its own segment.
// VEC: T % 256 == 0 and every array 16-byte aligned.
template <class Est, bool AGG, bool VEC, int OPT, class S = F32S>
__global__ void __launch_bounds__(256) seg_kernel(const KernelArgs p, int64_t seg_len, int64_t nseg) {
  using Tr = Traits<Est>;
  constexpr int K = 4;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;

  const int lane = threadIdx.x & 63;
  const int64_t T = p.T;
  const int64_t vrow = uniform64((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
  if (vrow >= p.E * nseg) return;  // (wave-uniform)
  const int64_t row = vrow / nseg;
  const int64_t seg = vrow - row * nseg;
  const int64_t t_begin = seg_begin(seg, seg_len);
  const int64_t t_end = seg_end(seg, seg_len, nseg, T);
  const int64_t ntl = (t_end - t_begin + kSegTile - 1) / kSegTile;
  const int64_t rb = row * T;  // element index of the row start
  const uint32_t last = (uint32_t)(T - 1);
  const bool first_lane = lane == 0;

  const double gamma = p.gamma, lam = p.lam;
  const ScanScalars sc{gamma, lam, gamma * lam, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0,
                       p.has_tboot != 0};
  const unsigned tmask = p.has_term ? ~0u : 0u;
  const unsigned rmask = p.has_trunc ? ~0u : 0u;
  const float rowv = p.has_row ? load1<S>(p.row, row, 0u) : 0.0f;
  const int64_t slot = rb + t_begin;  // element index of the segment's first output

  double C = 0.0;          // apply: value entering the current tile
  double A = 1.0, B = 0.0;  // aggregate: map of the tiles done so far
  if constexpr (!AGG) C = get_f64<S>(p.out0, slot);

  for (int64_t i = 0; i < ntl; ++i) {
    const int64_t tile_start = REV ? t_begin + (ntl - 1 - i) * kSegTile : t_begin + i * kSegTile;
    const int64_t cs64 = REV ? tile_start + kSegTile - (lane + 1) * K : tile_start + lane * K;
    const uint32_t cs = (uint32_t)cs64;
    const int64_t rem = T - cs64;
    const int nv = rem <= 0 ? 0 : (rem >= K ? K : (int)rem);

    LaneIn<Est, K> d;
    load_s<S, K, VEC>(p.r, rb, cs, last, d.s[0]);
    if constexpr (NS >= 2) load_s<S, K, VEC>(p.v, rb, cs, last, d.s[1]);
    if constexpr (NS >= 3) load_s<S, K, VEC>(p.aux, rb, cs, last, d.s[2]);
    if constexpr (NS >= 5) {
      load_s<S, K, VEC>(p.pi, rb, cs, last, d.s[3]);
      load_s<S, K, VEC>(p.mu, rb, cs, last, d.s[4]);
    }
    unsigned tbits = 0, rbits = 0;
    if constexpr (USE_FLAGS) {
      unsigned ft[K], fr[K];
      load_flag_raw<K, VEC>(p.term + rb, cs, last, ft);
      load_flag_raw<K, VEC>(p.trunc + rb, cs, last, fr);
      tbits = flag_bits<K, VEC>(ft) & tmask;
      rbits = flag_bits<K, VEC>(fr) & rmask;
    }
#pragma unroll
    for (int m = 0; m < K; ++m) d.tb[m] = 0.0f;
    if constexpr (GATHER_TB) {
      const unsigned need = rbits & ~tbits;
#pragma unroll
      for (int m = 0; m < K; ++m) {
        if ((need >> m) & 1u) {
          const uint32_t c = cs + m < last ? cs + m : last;
          d.tb[m] = load1<S>(p.tboot, rb, c);
        }
      }
    }
    d.rowv = rowv;

    // inputs of the scan predecessor of lane 0's innermost step (next tile or
    // previous tile of the row, possibly in another segment)
    const int64_t tn = REV ? tile_start + kSegTile : tile_start - 1;
    PredIn pred{0.0f, 0.0, 0u};
    if (tn >= 0 && tn < T) {
      const uint32_t n = (uint32_t)tn;
      if constexpr (Tr::kRetrace) {
        pred.v = load1<S>(p.aux, rb, n);
        const double ratio = (double)load1<S>(p.pi, rb, n) / (double)load1<S>(p.mu, rb, n);
        pred.c = lam * (ratio < 1.0 ? ratio : 1.0);
      } else if constexpr (Tr::kNbValue) {
        pred.v = load1<S>(p.v, rb, n);
      } else if constexpr (Tr::kNbDone && USE_FLAGS) {
        const unsigned dn = ((unsigned)(*at(p.term + rb, n) != 0) & tmask) |
                            ((unsigned)(*at(p.trunc + rb, n) != 0) & rmask);
        pred.done = dn ? 1u : 0u;
      }
    }

    // 16-bit formats: the fast Retrace quotient and V-trace exp (build_pairs)
    const LanePairs<K> lp = build_pairs<Est, K, VEC, !__is_same(S, F32S)>(d, sc, tbits, rbits, cs, T, nv, first_lane, pred);
    const AB incl = lane_scan<64>(fold_lane<K>(lp.e));
    if constexpr (AGG) {
      const double at_ = group_last_f64<64>(incl.a, lane);
      const double bt_ = group_last_f64<64>(incl.b, lane);
      B = __builtin_fma(at_, B, bt_);
      A = at_ * A;
    } else {
      const double y_last = __builtin_fma(incl.a, C, incl.b);
      const double from_below = shift_up_f64(y_last);
      const double x_in = first_lane ? C : from_below;
      const double C_next = group_last_f64<64>(y_last, lane);
      double xs[K];
      rewalk<K>(lp.e, x_in, xs);
      float o0[K], o1[K];
      epilogue<Est, K>(d, lp, sc, x_in, xs, o0, o1);
      store_s<S, K, VEC>(p.out0, rb, cs, nv, o0);
      if constexpr (OUT1) store_s<S, K, VEC>(p.out1, rb, cs, nv, o1);
      C = C_next;
    }
  }
  if constexpr (AGG) {
    if (first_lane) {
      put_f64<S>(p.out0, slot, A);
      put_f64<S>(p.out0, slot + f64_elems<S>(), B);
    }
  }
}

// Pass 2: one wave per row scans the segment maps in scan order, 64 at a time,
// and replaces each segment's (A, B) by the value entering it.  The value
// entering the row is 0 for the backward estimators (their bootstraps sit in
// the pairs) and the row's init / carry otherwise.
template <class Est, class S = F32S>
__global__ void __launch_bounds__(256) seg_carry_kernel(const KernelArgs p, int64_t seg_len, int64_t nseg) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
  const int lane = threadIdx.x & 63;
  const int64_t row = uniform64((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
  if (row >= p.E) return;  // (wave-uniform)
  double c = 0.0;
  if constexpr (!Tr::kBackwardRl) c = p.has_row ? (double)load1<S>(p.row, row, 0u) : 0.0;
  const int64_t base = row * p.T;
  for (int64_t k0 = 0; k0 < nseg; k0 += 64) {
    const int64_t k = k0 + lane;  // position in scan order
    const bool ok = k < nseg;
    const int64_t s = REV ? nseg - 1 - k : k;
    const int64_t slot = base + seg_begin(ok ? s : 0, seg_len);
    AB f{1.0, 0.0};
    if (ok) {
      f.a = get_f64<S>(p.out0, slot);
      f.b = get_f64<S>(p.out0, slot + f64_elems<S>());
    }
    const AB incl = lane_scan<64>(f);
    const double y = __builtin_fma(incl.a, c, incl.b);  // value leaving segment k
    const double from_below = shift_up_f64(y);
    const double cin = lane == 0 ? c : from_below;
    if (ok) put_f64<S>(p.out0, slot, cin);
    c = group_last_f64<64>(y, lane);
  }
}

}  // namespace rlscan
