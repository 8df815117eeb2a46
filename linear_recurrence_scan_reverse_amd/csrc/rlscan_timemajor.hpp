// rlscan_timemajor.hpp -- the estimators over time-major [T, E] arrays.
//
// Element (t, e) sits at t*E + e: one time step of every environment is
// contiguous, the order of rollout buffers that append one step for all
// environments at a time.  The recurrence and its pairs are those of the
// row-major kernels (gist.science summary of rl-triton, "Methodologie"
// sections 1 and 3); only the mapping to the machine changes.  The rl-triton
// skill page (skillsdirectory.com, "Implementation Workflow", step 2) lists
// the choice between contiguous and strided memory layouts among a kernel's
// settings; this is the strided one.
//
// Lanes map to environments: lane l of a block owns column e0 + l, so every
// load and store of one step is one coalesced run of 64 consecutive values.
// Time is cut into super-tiles of W x K steps; wave w owns the w-th chunk of
// K steps in scan order.  Each lane builds its K pairs with the per-lane code
// of the row-major kernels (a lane is its own team, and the scan predecessor
// of its chunk is loaded from memory), folds them into one affine map, and
// the W maps of a column meet in LDS: wave w composes the maps of the waves
// before it with the value entering the super-tile, rewalks its chunk from
// there and stores.  The composed map of all W chunks carries the column into
// the next super-tile.  Every input is read once (plus one predecessor step
// per chunk, which the neighbouring wave reads too) and every output written
// once; arithmetic is fp64 as everywhere else.  With few environments and
// long columns the columns are cut into segments scanned in three launches
// (MODE 1, tm_carry_kernel, MODE 2), which read the inputs twice.
#pragma once

#include "rlscan_kernel.hpp"
#include "rlscan_plan.hpp"

namespace rlscan {

// One element of format S at base[bidx + off], narrowed from fp32 (non-temporal).
template <class S>
__device__ __forceinline__ void store1(float* base, int64_t bidx, uint32_t off, float v) {
  if constexpr (__is_same(S, F32S)) __builtin_nontemporal_store(v, at(base + bidx, off));
  else __builtin_nontemporal_store(f32_to_s<S>(v), reinterpret_cast<uint16_t*>(base) + bidx + off);
}

// A double kept in a column of a time-major output: bit pieces in the
// column's elements at rows row0, row0 + 1, ... (two float32 rows, or four
// 16-bit rows).  Element (row, column e0 + lo) sits at row * E + e0 + lo.
template <class S>
constexpr int f64_rows() { return __is_same(S, F32S) ? 2 : 4; }
template <class S>
__device__ __forceinline__ void put_f64_col(float* out, int64_t row0, int64_t E, int64_t e0, uint32_t lo, double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
#pragma unroll
  for (int j = 0; j < f64_rows<S>(); ++j) {
    const int64_t i = (row0 + j) * E + e0 + lo;
    if constexpr (__is_same(S, F32S)) reinterpret_cast<uint32_t*>(out)[i] = (uint32_t)(u >> (32 * j));
    else reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)(u >> (16 * j));
  }
}
template <class S>
__device__ __forceinline__ double get_f64_col(const float* out, int64_t row0, int64_t E, int64_t e0, uint32_t lo) {
  unsigned long long u = 0;
#pragma unroll
  for (int j = 0; j < f64_rows<S>(); ++j) {
    const int64_t i = (row0 + j) * E + e0 + lo;
    if constexpr (__is_same(S, F32S)) u |= (unsigned long long)reinterpret_cast<const uint32_t*>(out)[i] << (32 * j);
    else u |= (unsigned long long)reinterpret_cast<const uint16_t*>(out)[i] << (16 * j);
  }
  return __builtin_bit_cast(double, u);
}

// W waves per block, K steps per wave chunk.  OPT as for scan_kernel.
//
// MODE 0 scans whole columns (block b: environments 64 b .. 64 b + 63).  With
// few environments and long rows that leaves most of the GPU idle, so time is
// cut into nseg segments of seg_len steps (the last takes the remainder) and
// scanned in three launches, as for long row-major rows: MODE 1 (block: one
// column group and one segment) composes the segment's steps into one affine
// map per column and parks it in the column's first output rows of the
// segment; tm_carry_kernel scans those maps per column and leaves the value
// entering each segment there; MODE 2 rescans every segment from that value
// and writes the outputs (overwriting the parked value).
template <class Est, int W, int K, int OPT, class S = F32S, int MODE = 0>
__global__ void __launch_bounds__(64 * W) tm_kernel(const KernelArgs p, int64_t seg_len, int64_t nseg) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  constexpr bool AGG = MODE == 1;
  constexpr int64_t SPAN = (int64_t)W * K;
  static_assert(!Tr::kDual, "one recurrence per pass");

  __shared__ double s_a[W][64];
  __shared__ double s_b[W][64];

  const int lane = threadIdx.x & 63;
  // chunk position in scan order inside a super-tile (wave-uniform)
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t E = p.E, T = p.T;
  const int64_t ngroups = (E + 63) / 64;
  const int64_t grp = MODE == 0 ? xcd_group(blockIdx.x, ngroups, 2) : (int64_t)blockIdx.x % ngroups;
  const int64_t sidx = MODE == 0 ? 0 : (int64_t)blockIdx.x / ngroups;
  // this block's steps [t0, t1)
  const int64_t t0 = MODE == 0 ? 0 : seg_begin(sidx, seg_len);
  const int64_t t1 = MODE == 0 ? T : seg_end(sidx, seg_len, nseg, T);
  // Addresses: a wave-uniform element index (step row + the block's first
  // column) plus a 32-bit lane offset, the lane's column clamped into the row
  // so every load stays inside the arrays.
  const int64_t e0 = grp * 64;
  const bool col_ok = e0 + lane < E;
  const uint32_t lo = (uint32_t)(col_ok ? lane : E - 1 - e0);

  const double gamma = p.gamma, lam = p.lam;
  const ScanScalars sc{gamma, lam, gamma * lam, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0,
                       p.has_tboot != 0};
  const unsigned tmask = p.has_term ? ~0u : 0u;
  const unsigned rmask = p.has_trunc ? ~0u : 0u;
  const float rowv = p.has_row ? load1<S>(p.row, e0, lo) : 0.0f;

  // value entering the current super-tile: 0 for the backward estimators (their
  // bootstraps sit in the pairs), the column's init / carry otherwise; in
  // MODE 2 the value the carry pass left for this segment (read by every wave
  // before the first barrier, so before any wave overwrites it)
  double C = 0.0;
  if constexpr (MODE == 0 && !Tr::kBackwardRl) C = p.has_row ? (double)rowv : 0.0;
  if constexpr (MODE == 2) C = get_f64_col<S>(p.out0, t0, E, e0, lo);
  double Am = 1.0, Bm = 0.0;  // MODE 1: map of the super-tiles done so far

  const int64_t nst = (t1 - t0 + SPAN - 1) / SPAN;
  for (int64_t s = 0; s < nst; ++s) {
    const int64_t tile = REV ? nst - 1 - s : s;
    const int64_t cs64 = REV ? t0 + tile * SPAN + SPAN - (int64_t)(w + 1) * K : t0 + tile * SPAN + (int64_t)w * K;
    const int64_t rem = t1 - cs64;
    const int nv = rem <= 0 ? 0 : (rem >= K ? K : (int)rem);
    const uint32_t cs = (uint32_t)cs64;  // T < 2^30

    LaneIn<Est, K> d;
    unsigned tbits = 0, rbits = 0;
#pragma unroll
    for (int m = 0; m < K; ++m) {
      const int64_t t = cs64 + m < T ? cs64 + m : T - 1;
      const int64_t row = t * E + e0;
      d.s[0][m] = load1<S>(p.r, row, lo);
      if constexpr (NS >= 2) d.s[1][m] = load1<S>(p.v, row, lo);
      if constexpr (NS >= 3) d.s[2][m] = load1<S>(p.aux, row, lo);
      if constexpr (NS >= 5) {
        d.s[3][m] = load1<S>(p.pi, row, lo);
        d.s[4][m] = load1<S>(p.mu, row, lo);
      }
      if constexpr (USE_FLAGS) {
        tbits |= (unsigned)(__builtin_nontemporal_load(at(p.term + row, lo)) != 0) << m;
        rbits |= (unsigned)(__builtin_nontemporal_load(at(p.trunc + row, lo)) != 0) << m;
      }
    }
    const unsigned vmask = nv >= 32 ? ~0u : ((1u << nv) - 1u);
    tbits &= tmask & vmask;
    rbits &= rmask & vmask;
#pragma unroll
    for (int m = 0; m < K; ++m) d.tb[m] = 0.0f;
    if constexpr (GATHER_TB) {
      const unsigned need = rbits & ~tbits;
#pragma unroll
      for (int m = 0; m < K; ++m)
        if ((need >> m) & 1u) d.tb[m] = load1<S>(p.tboot, (cs64 + m) * E + e0, lo);
    }
    d.rowv = rowv;

    // inputs of the scan predecessor of the chunk's innermost step (possibly
    // in the next or previous segment)
    const int64_t tn = REV ? cs64 + K : cs64 - 1;
    PredIn pred{0.0f, 0.0, 0u};
    if (tn >= 0 && tn < T) {
      const int64_t n = tn * E + e0;
      if constexpr (Tr::kRetrace) {
        pred.v = load1<S>(p.aux, n, lo);
        const double ratio = (double)load1<S>(p.pi, n, lo) / (double)load1<S>(p.mu, n, lo);
        pred.c = lam * (ratio < 1.0 ? ratio : 1.0);
      } else if constexpr (Tr::kNbValue) {
        pred.v = load1<S>(p.v, n, lo);
      } else if constexpr (Tr::kNbDone && USE_FLAGS) {
        const unsigned dn = ((unsigned)(*at(p.term + n, lo) != 0) & tmask) | ((unsigned)(*at(p.trunc + n, lo) != 0) & rmask);
        pred.done = dn ? 1u : 0u;
      }
    }

    // 16-bit formats: the fast Retrace quotient and V-trace exp (build_pairs)
    const LanePairs<K> lp = build_pairs<Est, K, false, !__is_same(S, F32S)>(d, sc, tbits, rbits, cs, T, nv, true, pred);
    const AB agg = fold_lane<K>(lp.e);
    s_a[w][lane] = agg.a;
    s_b[w][lane] = agg.b;
    __syncthreads();

    if constexpr (AGG) {
      // the super-tile's map (chunks in scan order), then the segment's so far
      double As = 1.0, Bs = 0.0;
      for (int u = 0; u < W; ++u) {
        Bs = __builtin_fma(s_a[u][lane], Bs, s_b[u][lane]);
        As = s_a[u][lane] * As;
      }
      Bm = __builtin_fma(As, Bm, Bs);
      Am = As * Am;
    } else {
      double x_in = C;  // value entering this wave's chunk
      for (int u = 0; u < w; ++u) x_in = __builtin_fma(s_a[u][lane], x_in, s_b[u][lane]);
      double c_out = x_in;  // value leaving the super-tile (the same in every wave)
      for (int u = w; u < W; ++u) c_out = __builtin_fma(s_a[u][lane], c_out, s_b[u][lane]);

      double xs[K];
      rewalk<K>(lp.e, x_in, xs);
      float o0[K], o1[K];
      epilogue<Est, K>(d, lp, sc, x_in, xs, o0, o1);
      if (col_ok) {
#pragma unroll
        for (int m = 0; m < K; ++m) {
          if (m < nv) {
            const int64_t row = (cs64 + m) * E + e0;
            store1<S>(p.out0, row, lo, o0[m]);
            if constexpr (OUT1) store1<S>(p.out1, row, lo, o1[m]);
          }
        }
      }
      C = c_out;
    }
    __syncthreads();  // the LDS maps are rewritten by the next super-tile
  }
  if constexpr (AGG) {
    if (w == 0 && col_ok) {
      put_f64_col<S>(p.out0, t0, E, e0, lo, Am);
      put_f64_col<S>(p.out0, t0 + f64_rows<S>(), E, e0, lo, Bm);
    }
  }
}

// Pass 2 of the segmented time-major path: one block of 16 waves per column
// group; wave w takes up to kTmCarrySeg consecutive segments (in scan order),
// composes their maps, the wave maps meet in LDS, and every wave then walks
// its segments from the value entering its first one, leaving each segment's
// entering value in place of its map.  nseg <= 16 * kTmCarrySeg.
template <class Est, class S = F32S>
__global__ void __launch_bounds__(1024) tm_carry_kernel(const KernelArgs p, int64_t seg_len, int64_t nseg) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
  constexpr int NW = 16;
  __shared__ double s_a[NW][64];
  __shared__ double s_b[NW][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t E = p.E;
  const int64_t e0 = (int64_t)blockIdx.x * 64;
  const bool col_ok = e0 + lane < E;
  const uint32_t lo = (uint32_t)(col_ok ? lane : E - 1 - e0);
  const int64_t q = (nseg + NW - 1) / NW;  // segments per wave (<= kTmCarrySeg)
  const int64_t k0 = (int64_t)w * q;      // first scan position of this wave

  double a[kTmCarrySeg], b[kTmCarrySeg];
  double Aw = 1.0, Bw = 0.0;
#pragma unroll
  for (int j = 0; j < kTmCarrySeg; ++j) {
    a[j] = 1.0;
    b[j] = 0.0;
    const int64_t k = k0 + j;
    if (j < q && k < nseg) {
      const int64_t sg = REV ? nseg - 1 - k : k;
      a[j] = get_f64_col<S>(p.out0, seg_begin(sg, seg_len), E, e0, lo);
      b[j] = get_f64_col<S>(p.out0, seg_begin(sg, seg_len) + f64_rows<S>(), E, e0, lo);
    }
  }
#pragma unroll
  for (int j = 0; j < kTmCarrySeg; ++j) {
    Bw = __builtin_fma(a[j], Bw, b[j]);
    Aw = a[j] * Aw;
  }
  s_a[w][lane] = Aw;
  s_b[w][lane] = Bw;
  __syncthreads();
  // value entering the column (0 for the backward estimators), then the waves before this one
  double c = 0.0;
  if constexpr (!Tr::kBackwardRl) c = p.has_row ? (double)load1<S>(p.row, e0, lo) : 0.0;
  for (int u = 0; u < w; ++u) c = __builtin_fma(s_a[u][lane], c, s_b[u][lane]);
#pragma unroll
  for (int j = 0; j < kTmCarrySeg; ++j) {
    const int64_t k = k0 + j;
    if (j < q && k < nseg) {
      const int64_t sg = REV ? nseg - 1 - k : k;
      if (col_ok) put_f64_col<S>(p.out0, seg_begin(sg, seg_len), E, e0, lo, c);
      c = __builtin_fma(a[j], c, b[j]);
    }
  }
}

}  // namespace rlscan
