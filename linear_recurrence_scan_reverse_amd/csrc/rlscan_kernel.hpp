// rlscan_kernel.hpp -- device side of librlscan (gfx950 / CDNA4, wave64).
//
// The pipelined kernel template solves every estimator as an affine scan.  The method
// (rl-triton; gist.science summary, "Methodologie" sections 1-2): each step t
// contributes a pair (a_t, b_t) such that x_t = a_t x_{t+1} + b_t (backward)
// or x_t = a_t x_{t-1} + b_t (forward); pairs compose associatively,
//     outer (+) inner = (a_o a_i, b_o + a_o b_i),
// where "inner" is the element nearer the scan's carry.  The pairs are built
// in registers from the raw inputs and never written to memory; every input
// element is read from HBM once and every output element written once.
//
// Work decomposition (ours, for 64-wide wavefronts):
//   * A row (one environment) is owned by a team: L = 16 or 32 lanes (several
//     rows per wave), one wave (L = 64), or W whole waves.
//   * The row is cut into tiles of SPAN = (lanes in team) * K steps; a lane
//     owns K consecutive steps of a tile (one 16-byte load per input when
//     K = 4).  Lanes are numbered in SCAN order: lane 0 holds the steps nearest
//     the carry (the latest steps for a backward scan), so a backward suffix
//     scan is an ordinary prefix scan over lane index while a wave still reads
//     one contiguous block of memory.
//   * Per tile ("item"): (1) each lane folds its K pairs serially; (2) a
//     log2(L)-step DPP prefix scan over lanes (row_shr 1,2,4,8, row_bcast 15,
//     row_bcast 31); (3) with W > 1 waves, wave totals meet in LDS; (4) each
//     lane takes its incoming value from its lower neighbour (DPP wave_shr 1)
//     and re-walks its K steps; (5) the epilogue forms the outputs and stores
//     them once.  The running value crosses tiles of a row in registers.
//   * Teams are persistent: each walks a sequence of items (the tiles of its
//     rows, in scan order) as a software pipeline -- flags are loaded two
//     items ahead, inputs one item ahead, and the gather of truncation
//     bootstraps (whose addresses depend on the flags) one item ahead, so
//     HBM latency overlaps the scan of the current item.  Every load is
//     branch-free: out-of-range elements read a clamped in-row address and
//     are masked in registers, so the compiler can count outstanding loads
//     exactly.
//   * One-item form (ONE = true, rows of one tile): the grid holds a team for
//     every row group; a team issues its flags and inputs together, gathers
//     the truncation bootstraps once the flags land, scans, stores and exits,
//     and the hardware refills the slot with the next block.  Nothing is
//     fetched ahead, so no pipeline has to fill or drain.
// All scan arithmetic is float64; inputs are float32 (or bfloat16 / float16,
// widened exactly) and each output is rounded to float32 once (then to the
// 16-bit format).  The per-lane code below (pairs, fold, re-walk, epilogue)
// is shared by every kernel of the library: this pipelined kernel, the
// streaming kernel, the segmented long-row path and the time-major kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlscan {

// ----------------------------------------------------------------- arguments
// Optional inputs are resolved on the host: a pointer below is never NULL when
// the kernel dereferences it; the has_* switches say whether its values count.
struct KernelArgs {
  const float* r;       // rewards; signal x (traces, prefix sums); a (generic scan)
  const float* v;       // values V; Q(s_t, a_t) (Retrace); b (generic scan)
  const float* aux;     // log_rhos (V-trace); E_pi Q(s_t, .) (Retrace)
  const float* pi;      // target-policy probability of a_t (Retrace)
  const float* mu;      // behaviour-policy probability of a_t (Retrace)
  const uint8_t* term;  // terminated flags (aliases `trunc` when absent)
  const uint8_t* trunc; // truncated flags (aliases `term` when absent)
  const float* row;     // [E]: bootstrap_value, init or carry (aliases r when absent)
  const float* tboot;   // [E,T] successor value at truncated steps (aliases r when absent)
  float* out0;          // main output
  float* out1;          // second output (GAE returns, V-trace pg); NULL = none
  int64_t E, T;
  double gamma, lam, rho_bar, c_bar;
  int has_term, has_trunc, has_row, has_tboot;
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
// Discounted return and TD(lambda) return of the same rollout in one pass.
struct ReturnsTdLambda { static constexpr bool kReverse = true; };

template <class Est> struct Traits {
  static constexpr bool kDual = __is_same(Est, ReturnsTdLambda);  // two recurrences per pass
  static constexpr bool kBackwardRl =
      __is_same(Est, DiscountedReturn) || __is_same(Est, TdLambda) || __is_same(Est, Gae) ||
      __is_same(Est, Vtrace) || __is_same(Est, Retrace) || kDual;
  static constexpr bool kForwardRl = __is_same(Est, EligibilityTrace) || __is_same(Est, EpisodicPrefixSum);
  static constexpr bool kLinear = __is_same(Est, LinearScanReverse) || __is_same(Est, LinearScanForward);
  static constexpr bool kRetrace = __is_same(Est, Retrace);
  static constexpr bool kVtrace = __is_same(Est, Vtrace);
  // float input streams: 0 = r, 1 = v/q/b, 2 = aux, 3 = pi, 4 = mu
  static constexpr int kStreams = kRetrace ? 5 : kVtrace ? 3
                                  : (__is_same(Est, TdLambda) || __is_same(Est, Gae) || kLinear || kDual) ? 2 : 1;
  static constexpr bool kUsesFlags = kBackwardRl || kForwardRl || kLinear;  // (linear: episode cuts)
  // value handed from a step to its scan-successor: V (TD, GAE, V-trace), EQ and c (Retrace)
  static constexpr bool kNbValue = __is_same(Est, TdLambda) || __is_same(Est, Gae) || kVtrace || kRetrace || kDual;
  static constexpr bool kNbDone = kForwardRl || __is_same(Est, LinearScanForward);  // previous step's done flag
  static constexpr bool kHasOut1 = __is_same(Est, Gae) || kVtrace || kDual;
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

// 32-bit DPP move whose source-less lanes read 0 (bound_ctrl), so no `old`
// value has to be materialised; valid only with every row enabled.
template <int CTRL>
__device__ __forceinline__ int dpp_zero(int src) {
  return __builtin_amdgcn_update_dpp(0, src, CTRL, 0xf, 0xf, true);
}

// The pair of lane (i - shift) or the identity element (1, 0) where the source
// lane is missing (or its row masked off).  Words of the identity that are 0
// come from bound_ctrl's zero fill; only the high word of a = 1.0 needs `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ AB dpp_ab(const AB& v) {
  AB r;
  if constexpr (ROW_MASK == 0xf) {
    const unsigned long long ua = __builtin_bit_cast(unsigned long long, v.a);
    const unsigned long long ub = __builtin_bit_cast(unsigned long long, v.b);
    const unsigned alo = (unsigned)dpp_zero<CTRL>((int)(unsigned)ua);
    const unsigned ahi = (unsigned)__builtin_amdgcn_update_dpp((int)0x3ff00000, (int)(unsigned)(ua >> 32), CTRL,
                                                               0xf, 0xf, false);
    const unsigned blo = (unsigned)dpp_zero<CTRL>((int)(unsigned)ub);
    const unsigned bhi = (unsigned)dpp_zero<CTRL>((int)(unsigned)(ub >> 32));
    r.a = __builtin_bit_cast(double, ((unsigned long long)ahi << 32) | alo);
    r.b = __builtin_bit_cast(double, ((unsigned long long)bhi << 32) | blo);
  } else {
    r.a = dpp_f64<CTRL, ROW_MASK>(1.0, v.a);
    r.b = dpp_f64<CTRL, ROW_MASK>(0.0, v.b);
  }
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
__device__ __forceinline__ unsigned shift_up_u32(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xf, 0xf, false);
}

// Broadcast of lane (group start + L - 1) to the group.
// Retrace trace coefficient c = lam * min(1, pi / mu) without an fp64
// division: the fp32 reciprocal of mu (good to about 1e-7) refined by one
// Newton step in fp64, which squares its error (about 1e-14), times pi.  Used
// by the 16-bit storage formats, where the pipelined kernel is bound by vector
// instructions: at 16384 x 256 Retrace in bfloat16 ran 16.4 -> 15.3 us.  In
// float32 the kernel streams at its byte mix's speed and the fp64 division
// measured 0.15-0.7 us faster, so float32 keeps it.  mu = 0 (or a denormal)
// gives a NaN quotient and so c = lam, as pi / 0 = inf does with the division.
__device__ __forceinline__ double retrace_c_fast(double lam, float pi, float mu) {
  const double m = (double)mu;
  const double r0 = (double)__builtin_amdgcn_rcpf(mu);
  const double r1 = __builtin_fma(r0, __builtin_fma(-m, r0, 1.0), r0);
  const double ratio = (double)pi * r1;
  return lam * (ratio < 1.0 ? ratio : 1.0);
}

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

// Column group of block b of n, for kernels whose neighbouring column groups
// share 128-byte lines of the flag arrays (R groups per line: a flag row of a
// group is 128 / R bytes).  Blocks go to the 8 XCDs of the chip round-robin,
// and each XCD has its own L2, so groups g and g + 1 on different XCDs each
// fetch their shared lines from HBM; here the R groups of a line go to the
// same XCD.  Bijective on [0, n): blocks past the last whole set of 8 R keep
// their own group.
__device__ __forceinline__ int64_t xcd_group(int64_t b, int64_t n, int R) {
  const int64_t span = 8 * (int64_t)R;
  if (b >= n / span * span) return b;
  const int64_t x = b % 8, i = b / 8;
  return span * (i / R) + R * x + i % R;
}

// ----------------------------------------------------------------- streaming loads / stores
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every [E,T] array is addressed as (wave-uniform base pointer) + (32-bit lane
// offset in elements); all arrays share one layout, so one offset register
// serves every stream and the loads use the scalar-base addressing mode.

// base + off elements, formed as a 32-bit byte offset so the compiler can use
// the scalar-base + 32-bit vector-offset addressing mode.
__device__ __forceinline__ const float* at(const float* base, uint32_t off) {
  return reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + (uint32_t)(off * 4u));
}
__device__ __forceinline__ float* at(float* base, uint32_t off) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(base) + (uint32_t)(off * 4u));
}
__device__ __forceinline__ const uint8_t* at(const uint8_t* base, uint32_t off) { return base + off; }

// K consecutive floats at base[off].  VEC: one aligned vector load (the whole
// chunk lies inside its row); otherwise each element is read at its column
// clamped into the row (`last` = offset of the row's last element), so the
// address is always valid.
template <int K, bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ base, uint32_t off, uint32_t last,
                                           float (&o)[K]) {
  if constexpr (VEC) {
    if constexpr (K == 1) {
      o[0] = __builtin_nontemporal_load(at(base, off));
    } else if constexpr (K == 2) {
      const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(at(base, off)));
      o[0] = t.x; o[1] = t.y;
    } else if constexpr (K == 4) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(at(base, off)));
      o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
    } else {
      static_assert(K == 8, "chunk");
      const f32x4 t0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(at(base, off)));
      const f32x4 t1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(at(base, off + 4)));
      o[0] = t0.x; o[1] = t0.y; o[2] = t0.z; o[3] = t0.w;
      o[4] = t1.x; o[5] = t1.y; o[6] = t1.z; o[7] = t1.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m) {
      const uint32_t c = off + m < last ? off + m : last;
      o[m] = __builtin_nontemporal_load(at(base, c));
    }
  }
}

// K flag bytes at base[off], loaded raw (decoded only when the item is
// computed, so the loads stay in flight): VEC with K >= 4 reads K/4 dwords,
// otherwise each byte is read at its clamped column.
template <int K> struct FlagRaw {
  unsigned t[K], r[K];
};

template <int K, bool VEC>
__device__ __forceinline__ void load_flag_raw(const uint8_t* __restrict__ base, uint32_t off, uint32_t last,
                                              unsigned (&o)[K]) {
  if constexpr (VEC && K >= 4) {
#pragma unroll
    for (int i = 0; i < K / 4; ++i)
      o[i] = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(at(base, off + 4 * i)));
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m) {
      const uint32_t c = off + m < last ? off + m : last;
      o[m] = __builtin_nontemporal_load(at(base, c));
    }
  }
}

// Packed flag words (4 bytes each) to a bit mask: bit 4i+b is set iff byte b
// of word i is nonzero.
template <int NW>
__device__ __forceinline__ unsigned flag_bits_words(const unsigned* w) {
  unsigned bits = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    // bit 7 of each byte of nz is set iff that byte is nonzero
    const unsigned nz = (((w[i] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[i]) & 0x80808080u;
    const unsigned b4 = ((nz >> 7) & 1u) | ((nz >> 14) & 2u) | ((nz >> 21) & 4u) | ((nz >> 28) & 8u);
    bits |= b4 << (4 * i);
  }
  return bits;
}

// Bit m of the result is set iff flag byte m is nonzero.
template <int K, bool VEC>
__device__ __forceinline__ unsigned flag_bits(const unsigned (&o)[K]) {
  unsigned bits = 0;
  if constexpr (VEC && K >= 4) {
    bits = flag_bits_words<K / 4>(o);
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m) bits |= (unsigned)(o[m] != 0) << m;
  }
  return bits;
}

template <int K, bool VEC>
__device__ __forceinline__ void store_chunk(float* __restrict__ base, uint32_t off, int nv, const float (&o)[K]) {
  if constexpr (VEC) {
    if constexpr (K == 1) {
      __builtin_nontemporal_store(o[0], at(base, off));
    } else if constexpr (K == 2) {
      __builtin_nontemporal_store((f32x2){o[0], o[1]}, reinterpret_cast<f32x2*>(at(base, off)));
    } else if constexpr (K == 4) {
      __builtin_nontemporal_store((f32x4){o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(at(base, off)));
    } else {
      __builtin_nontemporal_store((f32x4){o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(at(base, off)));
      __builtin_nontemporal_store((f32x4){o[4], o[5], o[6], o[7]}, reinterpret_cast<f32x4*>(at(base, off + 4)));
    }
  } else {
#pragma unroll
    for (int m = 0; m < K; ++m)
      if (m < nv) __builtin_nontemporal_store(o[m], at(base, off + m));
  }
}

// ----------------------------------------------------------------- storage formats
// Values live in HBM as fp32 (the default) or as 16-bit bf16 / fp16; they are
// widened on load and the fp64 results rounded once to fp32, then (16-bit
// formats) to the storage format, round to nearest even.  Kernel arguments keep
// `const float*` fields; for 16-bit formats they address 16-bit elements.
struct F32S {
  using T = float;
};
struct Bf16S {
  using T = uint16_t;
};
struct F16S {
  using T = uint16_t;
};

template <class S>
__device__ __forceinline__ float s_to_f32(typename S::T v) {
  if constexpr (__is_same(S, F32S)) return v;
  else if constexpr (__is_same(S, Bf16S)) return __builtin_bit_cast(float, (uint32_t)v << 16);
  else return (float)__builtin_bit_cast(_Float16, v);
}
template <class S>
__device__ __forceinline__ typename S::T f32_to_s(float v) {
  // round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_f16_f32).  The empty asm
  // keeps v a float32: without it the compiler folds the earlier fp64 -> fp32
  // rounding and this one into a single fp64 -> fp16 rounding (a long
  // software sequence, and not the documented two roundings).
  if constexpr (__is_same(S, F32S)) {
    return v;
  } else {
    __asm__("" : "+v"(v));
    if constexpr (__is_same(S, Bf16S)) return __builtin_bit_cast(uint16_t, (__bf16)v);
    else return __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

// One element: base[bidx + off], widened.
template <class S>
__device__ __forceinline__ float load1(const float* base, int64_t bidx, uint32_t off) {
  if constexpr (__is_same(S, F32S)) return __builtin_nontemporal_load(at(base + bidx, off));
  else return s_to_f32<S>(__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(base) + bidx + off));
}

// K consecutive elements at base[bidx + off] (same contract as load_chunk).
template <class S, int K, bool VEC>
__device__ __forceinline__ void load_s(const float* base, int64_t bidx, uint32_t off, uint32_t last,
                                       float (&o)[K]) {
  if constexpr (__is_same(S, F32S)) {
    load_chunk<K, VEC>(base + bidx, off, last, o);
  } else {
    const uint16_t* b = reinterpret_cast<const uint16_t*>(base) + bidx;
    if constexpr (VEC && K == 8) {
      // integer loads: a float-vector load of these bits was narrowed to one
      // dword by the compiler
      const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + off));
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = s_to_f32<S>((uint16_t)w[i]);
        o[2 * i + 1] = s_to_f32<S>((uint16_t)(w[i] >> 16));
      }
    } else if constexpr (VEC && K == 4) {
      const unsigned long long q = __builtin_nontemporal_load(reinterpret_cast<const unsigned long long*>(b + off));
      const uint32_t w0 = (uint32_t)q, w1 = (uint32_t)(q >> 32);
      o[0] = s_to_f32<S>((uint16_t)w0); o[1] = s_to_f32<S>((uint16_t)(w0 >> 16));
      o[2] = s_to_f32<S>((uint16_t)w1); o[3] = s_to_f32<S>((uint16_t)(w1 >> 16));
    } else if constexpr (VEC && K == 2) {
      const uint32_t w0 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(b + off));
      o[0] = s_to_f32<S>((uint16_t)w0); o[1] = s_to_f32<S>((uint16_t)(w0 >> 16));
    } else {
#pragma unroll
      for (int m = 0; m < K; ++m) {
        const uint32_t c = off + m < last ? off + m : last;
        o[m] = s_to_f32<S>(__builtin_nontemporal_load(b + c));
      }
    }
  }
}

// K consecutive outputs at base[bidx + off] (same contract as store_chunk).
template <class S, int K, bool VEC>
__device__ __forceinline__ void store_s(float* base, int64_t bidx, uint32_t off, int nv, const float (&o)[K]) {
  if constexpr (__is_same(S, F32S)) {
    store_chunk<K, VEC>(base + bidx, off, nv, o);
  } else {
    uint16_t* b = reinterpret_cast<uint16_t*>(base) + bidx;
    if constexpr (VEC && K == 8) {
      u32x4 q;
      q.x = (uint32_t)f32_to_s<S>(o[0]) | ((uint32_t)f32_to_s<S>(o[1]) << 16);
      q.y = (uint32_t)f32_to_s<S>(o[2]) | ((uint32_t)f32_to_s<S>(o[3]) << 16);
      q.z = (uint32_t)f32_to_s<S>(o[4]) | ((uint32_t)f32_to_s<S>(o[5]) << 16);
      q.w = (uint32_t)f32_to_s<S>(o[6]) | ((uint32_t)f32_to_s<S>(o[7]) << 16);
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(b + off));
    } else if constexpr (VEC && K == 4) {
      const uint32_t w0 = (uint32_t)f32_to_s<S>(o[0]) | ((uint32_t)f32_to_s<S>(o[1]) << 16);
      const uint32_t w1 = (uint32_t)f32_to_s<S>(o[2]) | ((uint32_t)f32_to_s<S>(o[3]) << 16);
      __builtin_nontemporal_store((unsigned long long)w0 | ((unsigned long long)w1 << 32),
                                  reinterpret_cast<unsigned long long*>(b + off));
    } else if constexpr (VEC && K == 2) {
      const uint32_t w0 = (uint32_t)f32_to_s<S>(o[0]) | ((uint32_t)f32_to_s<S>(o[1]) << 16);
      __builtin_nontemporal_store(w0, reinterpret_cast<uint32_t*>(b + off));
    } else {
#pragma unroll
      for (int m = 0; m < K; ++m)
        if (m < nv) __builtin_nontemporal_store(f32_to_s<S>(o[m]), b + off + m);
    }
  }
}

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ----------------------------------------------------------------- one row tile, one lane
// The estimator-specific part of the scan, shared by both kernels: from one
// lane's K raw steps to its K pairs (a_t, b_t), and from the scanned values
// x_t back to the outputs.

// Inputs of one lane's chunk of one row tile.
template <class Est, int K> struct LaneIn {
  float s[Traits<Est>::kStreams][K];  // raw inputs, memory order
  float tb[K];                        // truncation bootstraps (valid where truncated)
  float rowv;                         // bootstrap / init / carry of the row
};

// Scalars of a call.
struct ScanScalars {
  double gamma, lam, gl;  // gl = gamma * lambda
  float rho_bar, c_bar;
  bool has_row, has_tboot;
};

// Inputs of the scan predecessor of the team-first lane's innermost step
// (it lives in another wave, team slot or tile).
struct PredIn {
  float v;        // V_{t+1} (TD, GAE, V-trace) or EQ_{t+1} (Retrace)
  double c;       // c_{t+1} (Retrace)
  unsigned done;  // done_{t-1} (forward estimators)
};

// Per-lane result of building the pairs.
template <int K> struct LanePairs {
  AB e[K];           // pairs in scan order (j = 0 nearest the carry)
  float rho[K];      // V-trace: rho_t (a float32 value; widened where used)
  float succv[K];    // V-trace: the cut's successor value (a float32 input)
  unsigned cut;      // K-bit mask of steps after which the episode chain stops
  float nb_v;        // value handed in for the innermost step (V-trace epilogue)
};

// Build the K pairs of one lane.  cs: column of the lane's lowest-addressed
// step; nv: steps inside the row (VEC: always K); tbits / rbits: terminated /
// truncated bit masks (bit m = memory index m).
// FASTDIV: Retrace's quotient pi / mu by retrace_c_fast instead of an fp64
// division (V-trace's exp is the hardware one in every format).
template <class Est, int K, bool VEC, bool FASTDIV = false>
__device__ __forceinline__ LanePairs<K> build_pairs(const LaneIn<Est, K>& d, const ScanScalars& sc, unsigned tbits,
                                                    unsigned rbits, uint32_t cs, int64_t T, int nv,
                                                    bool team_first_lane, const PredIn& pred) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
  constexpr int MLAST = REV ? 0 : K - 1;  // memory index of the lane's outermost step
  LanePairs<K> out;
  const double gamma = sc.gamma, lam = sc.lam, gl = sc.gl;

  // ---- step kinds as K-bit lane masks
  const unsigned te = tbits;                    // terminated
  const unsigned trm = rbits & ~te;             // truncated (terminated wins)
  unsigned endm = 0;                            // plain window end, t = T - 1
  {
    const int64_t e_m = T - 1 - (int64_t)cs;
    if (e_m >= 0 && e_m < K) endm = (1u << e_m) & ~te & ~trm;
  }
  const unsigned cut = te | trm | endm;
  const unsigned trb = sc.has_tboot ? trm : 0u;  // truncations with a supplied bootstrap
  const float brow = sc.has_row ? d.rowv : 0.0f;
  out.cut = cut;

  // ---- scan-predecessor values for the lane's innermost step
  double cown[K];
  if constexpr (Tr::kRetrace) {
#pragma unroll
    for (int m = 0; m < K; ++m) {
      if constexpr (FASTDIV) {
        cown[m] = retrace_c_fast(lam, d.s[3][m], d.s[4][m]);
      } else {
        const double ratio = (double)d.s[3][m] / (double)d.s[4][m];
        cown[m] = lam * (ratio < 1.0 ? ratio : 1.0);
      }
    }
  }
  float nb_v = 0.0f;
  double nb_c = 0.0;
  unsigned nb_done = 0;
  if constexpr (Tr::kNbValue) {
    nb_v = shift_up_f32(Tr::kRetrace ? d.s[2][MLAST] : d.s[1][MLAST]);
    if constexpr (Tr::kRetrace) nb_c = shift_up_f64(cown[MLAST]);
  }
  if constexpr (Tr::kNbDone) nb_done = shift_up_u32(((tbits | rbits) >> MLAST) & 1u);
  if (team_first_lane) {
    nb_v = pred.v;
    nb_c = pred.c;
    nb_done = pred.done;
  }
  out.nb_v = nb_v;

  // ---- pairs, scan order j = 0..K-1
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int m = REV ? (K - 1 - j) : j;
    AB c;
    out.rho[j] = 0.0f;
    out.succv[j] = 0.0f;
    if constexpr (Tr::kBackwardRl) {
      const bool is_cut = (cut >> m) & 1u;
      // successor value at a cut (0 terminated / trunc bootstrap / row bootstrap)
      const float bvf = ((trb >> m) & 1u) ? d.tb[m] : (((endm >> m) & 1u) ? brow : 0.0f);
      float vnx = 0.0f;  // raw next-step input (V or EQ) in the same episode
      double cn = 0.0;
      if constexpr (Tr::kNbValue) {
        if (j == 0) {
          vnx = nb_v;
          if constexpr (Tr::kRetrace) cn = nb_c;
        } else {
          const int mp = REV ? m + 1 : m - 1;
          vnx = Tr::kRetrace ? d.s[2][mp] : d.s[1][mp];
          if constexpr (Tr::kRetrace) cn = cown[mp];
        }
      }
      const double nu = (double)(is_cut ? bvf : vnx);  // successor value
      const double r = (double)d.s[0][m];
      if constexpr (__is_same(Est, DiscountedReturn)) {
        c.a = is_cut ? 0.0 : gamma;
        c.b = __builtin_fma(gamma, (double)bvf, r);  // bvf is 0 off cuts
      } else if constexpr (__is_same(Est, TdLambda)) {
        c.a = is_cut ? 0.0 : gl;
        c.b = __builtin_fma(is_cut ? gamma : (gamma - gl), nu, r);  // r + g((1-l) V' or boot)
      } else if constexpr (__is_same(Est, Gae)) {
        c.a = is_cut ? 0.0 : gl;
        c.b = __builtin_fma(gamma, nu, r) - (double)d.s[1][m];
      } else if constexpr (Tr::kVtrace) {
        // e^x as the hardware exp2 of x log2(e) in every format: relative error
        // about (|x| + 1) 2^-24 (the rounding of the product, one unit of the
        // exp2).  With clips at 1 (rho_bar, c_bar) only x < 0 reaches an output,
        // where the error of e^x is at most |x| e^x 2^-24 < 2.2e-8 absolute.
        // Against the libm expf, float32 V-trace 16384 x 256 18.35 -> 17.92 us
        // (bfloat16 16.4 -> 15.6 when that format took it first).
        const float ratio = __expf(d.s[2][m]);
        const float rhf = fminf(ratio, sc.rho_bar);
        const double rh = (double)rhf;
        const double ct = (double)fminf(ratio, sc.c_bar);
        c.a = is_cut ? 0.0 : gl * ct;
        c.b = rh * (__builtin_fma(gamma, nu, r) - (double)d.s[1][m]);
        out.rho[j] = rhf;
        out.succv[j] = bvf;
      } else if constexpr (Tr::kRetrace) {
        c.a = is_cut ? 0.0 : gamma * cn;
        c.b = __builtin_fma(gamma, nu, r) - (double)d.s[1][m];
      }
    } else if constexpr (Tr::kForwardRl) {
      // keep the running value unless the previous step ended an episode
      const unsigned prev_done = (j == 0) ? nb_done : (((tbits | rbits) >> (m - 1)) & 1u);
      const bool keep = !prev_done || (cs + m == 0);
      if constexpr (__is_same(Est, EligibilityTrace)) c.a = keep ? gl : 0.0;
      else c.a = keep ? 1.0 : 0.0;
      c.b = (double)d.s[0][m];
    } else {
      // generic recurrence; a flagged step cuts the chain: backward, nothing
      // enters step t from t+1; forward, nothing enters step t from t-1
      bool keep = true;
      if constexpr (REV) {
        keep = !(((tbits | rbits) >> m) & 1u);
      } else {
        const unsigned prev_done = (j == 0) ? nb_done : (((tbits | rbits) >> (m - 1)) & 1u);
        keep = !prev_done || (cs + m == 0);
      }
      c.a = keep ? (double)d.s[0][m] : 0.0;
      c.b = (double)d.s[1][m];
    }
    if constexpr (!VEC) {
      if (m >= nv) c = AB{1.0, 0.0};  // past the row end: identity
    }
    out.e[j] = c;
  }
  return out;
}

// Serial fold of the lane's K pairs (outermost applied last).
template <int K>
__device__ __forceinline__ AB fold_lane(const AB (&e)[K]) {
  AB agg = e[0];
#pragma unroll
  for (int j = 1; j < K; ++j) agg = compose(e[j], agg);
  return agg;
}

// Re-walk the lane's K steps from the value entering it.
template <int K>
__device__ __forceinline__ void rewalk(const AB (&e)[K], double x_in, double (&xs)[K]) {
  double x = x_in;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    x = __builtin_fma(e[j].a, x, e[j].b);
    xs[j] = x;
  }
}

// Outputs of the lane's K steps (memory order), rounded once to fp32.
template <class Est, int K>
__device__ __forceinline__ void epilogue(const LaneIn<Est, K>& d, const LanePairs<K>& lp, const ScanScalars& sc,
                                         double x_in, const double (&xs)[K], float (&o0)[K], float (&o1)[K]) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int m = REV ? (K - 1 - j) : j;
    double y = xs[j];
    double y1 = 0.0;
    if constexpr (__is_same(Est, Gae)) {
      y1 = y + (double)d.s[1][m];
    } else if constexpr (Tr::kVtrace) {
      // pg_t = rho_t (r_t + gamma vs_{t+1} - V_t); vs_{t+1} = V_{t+1} + x_{t+1} inside
      // the episode, the cut's successor value otherwise
      const double xprev = (j == 0) ? x_in : xs[j - 1];
      const int mp = REV ? m + 1 : m - 1;
      const float vnx = (j == 0) ? lp.nb_v : d.s[1][(mp < 0 || mp >= K) ? 0 : mp];
      const double succ = ((lp.cut >> m) & 1u) ? (double)lp.succv[j] : ((double)vnx + xprev);
      y1 = (double)lp.rho[j] * (__builtin_fma(sc.gamma, succ, (double)d.s[0][m]) - (double)d.s[1][m]);
      y = (double)d.s[1][m] + y;
    } else if constexpr (Tr::kRetrace) {
      y = (double)d.s[1][m] + y;
    }
    o0[m] = (float)y;
    o1[m] = (float)y1;
  }
}

// ----------------------------------------------------------------- per-item registers
// An item is one tile of R rows.  Its lane-level position within the tile is
// the same for all R rows.
struct TilePos {
  uint32_t cs;  // column of this lane's lowest-addressed step
  uint32_t tn;  // column of the team-first lane's scan predecessor, clamped into the row
  int nv;       // steps of this lane's chunk that lie inside the row (0..K)
  bool nb_ok;   // the scan predecessor of the team-first lane exists
  bool first;   // first tile of its rows in scan order
};

// The item's rows: a wave-uniform base row plus, per row, the element offset
// of the row start relative to that base.
template <int R> struct ItemRows {
  int64_t wb;        // base row (uniform across the wave)
  uint32_t roff[R];  // (row - wb) * T, rows clamped to E - 1
  uint32_t rsel[R];  // row - wb
  bool ok[R];        // the row exists
};

template <class Est, int K> struct RowData : LaneIn<Est, K> {
  float nb[3];       // raw inputs of the team-first lane's scan predecessor
  unsigned nbf[2];   // its raw terminated / truncated bytes (forward estimators)
};

// ----------------------------------------------------------------- the kernel
// Template parameters: estimator tag, team width L (lanes per row when W = 1),
// chunk K (steps per lane per tile), W (waves per row; W > 1 requires L = 64),
// R (rows a team scans side by side per item: more bytes in flight per wave),
// VEC (rows aligned for K-wide vector accesses and T % SPAN == 0, so every
// tile is whole; otherwise every element is loaded at a clamped column), OPT
// (bit 0: a flag array is present; bit 1: the second output is written).
// The C ABI guarantees T < 2^30, so every in-row byte offset fits 32 bits.
template <class Est, int L, int K, int W, int R, bool VEC, int OPT, class S = F32S, bool ONE = false>
__global__ void __launch_bounds__(BlockShape<W>::kThreads)
scan_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr bool REV = Est::kReverse;
  constexpr int BLOCK = BlockShape<W>::kThreads;
  constexpr int TEAM_LANES = (W > 1) ? 64 * W : L;
  constexpr int TEAMS = BLOCK / TEAM_LANES;
  constexpr int SPAN = TEAM_LANES * K;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  static_assert(W == 1 || L == 64, "multi-wave teams use full waves");
  static_assert(BLOCK % TEAM_LANES == 0, "block shape");

  __shared__ double s_tot[(W > 1) ? 2 : 1][TEAMS][R][(W > 1) ? W : 1][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int team = tid / TEAM_LANES;
  const int w = (W > 1) ? ((tid >> 6) % W) : 0;     // wave inside the team (0 = nearest the carry)
  const int g = (W > 1) ? lane : (lane & (L - 1));  // lane inside this wave's part of the team
  const int team_in_wave = (W > 1) ? 0 : lane / L;  // teams sharing this wave, in lane order
  const bool team_first_lane = (g == 0);            // scan predecessor lives outside this wave
  const int pos0 = (w * 64 + g) * K;                // scan position of this lane's innermost step

  const int64_t T = p.T;
  const int64_t E = p.E;
  const uint32_t T32 = (uint32_t)T;
  const int64_t ntiles = (T + SPAN - 1) / SPAN;
  const int64_t groups = (E + R - 1) / R;  // row groups of R consecutive rows
  const int64_t teams_total = (int64_t)gridDim.x * TEAMS;
  const int64_t my_team = (int64_t)blockIdx.x * TEAMS + team;
  // Block-uniform item count: the block's first team has the most row groups.
  const int64_t first_team = (int64_t)blockIdx.x * TEAMS;
  // In Retrace's one-item form the grid holds a team for every row group, so a
  // comparison gives the count.  Measured on one MI355X at 16384 x 256 (two
  // runs each): Retrace 20.7 -> 20.2 us without the 64-bit division, while
  // V-trace's one-item form ran 0.15 us slower without it and keeps it.
  constexpr bool kCountByCompare = ONE && Tr::kRetrace;
  const int64_t groups_first =
      first_team >= groups ? 0
                           : (kCountByCompare ? 1 : (groups - first_team + teams_total - 1) / teams_total);
  const int64_t n_items = groups_first * ntiles;

  const double gamma = p.gamma;
  const double lam = p.lam;
  const double gl = gamma * lam;
  const unsigned tmask = p.has_term ? ~0u : 0u;
  const unsigned rmask = p.has_trunc ? ~0u : 0u;

  // ---------------------------------------------------------------- item cursors
  // An item is (j, ts): the j-th row group of this team, ts-th tile in scan order.
  struct Cursor {
    int64_t k, j, ts;
  };
  auto advance = [&](Cursor c) __attribute__((always_inline)) {
    c.k += 1;
    c.ts += 1;
    if (c.ts == ntiles) {
      c.ts = 0;
      c.j += 1;
    }
    return c;
  };
  auto tile_pos = [&](const Cursor& c) __attribute__((always_inline)) {
    TilePos q;
    const uint32_t tile = (uint32_t)(REV ? (ntiles - 1 - c.ts) : c.ts);
    const uint32_t tile_start = tile * (uint32_t)SPAN;
    q.cs = REV ? (tile_start + SPAN - pos0 - K) : (tile_start + pos0);
    const int rem = (int)((int64_t)T - (int64_t)q.cs);
    q.nv = rem <= 0 ? 0 : (rem >= K ? K : rem);
    const int64_t cs0 = REV ? (int64_t)tile_start + SPAN - w * 64 * K - K : (int64_t)tile_start + w * 64 * K;
    const int64_t tn = REV ? (cs0 + K) : (cs0 - 1);
    q.nb_ok = tn >= 0 && tn < T;
    q.tn = (uint32_t)(tn < 0 ? 0 : (tn >= T ? T - 1 : tn));
    q.first = (c.ts == 0);
    return q;
  };
  auto item_rows = [&](const Cursor& c) __attribute__((always_inline)) {
    ItemRows<R> ir;
    const int64_t grp = my_team + c.j * teams_total;
    const int64_t wave_grp = grp - team_in_wave;  // this wave's first team
    int64_t wb = wave_grp * R;
    wb = wb < E ? wb : E - 1;
    ir.wb = uniform64(wb);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int64_t row = grp * R + rr;
      ir.ok[rr] = (c.k < n_items) && row < E;
      const int64_t rc = row < E ? row : E - 1;
      ir.rsel[rr] = (uint32_t)(rc - ir.wb);
      ir.roff[rr] = ir.rsel[rr] * T32;
    }
    return ir;
  };

  // ---------------------------------------------------------------- pipeline stages
  auto issue_flags = [&](const Cursor& c, FlagRaw<K> (&f)[R]) __attribute__((always_inline)) {
    if constexpr (USE_FLAGS) {
      const TilePos q = tile_pos(c);
      const ItemRows<R> ir = item_rows(c);
      const uint8_t* tb = p.term + ir.wb * T;
      const uint8_t* rb = p.trunc + ir.wb * T;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const uint32_t last = ir.roff[rr] + T32 - 1;
        load_flag_raw<K, VEC>(tb, ir.roff[rr] + q.cs, last, f[rr].t);
        load_flag_raw<K, VEC>(rb, ir.roff[rr] + q.cs, last, f[rr].r);
      }
    }
  };

  auto decode = [&](const FlagRaw<K> (&f)[R], unsigned (&tbits)[R], unsigned (&rbits)[R])
      __attribute__((always_inline)) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      tbits[rr] = 0;
      rbits[rr] = 0;
      if constexpr (USE_FLAGS) {
        tbits[rr] = flag_bits<K, VEC>(f[rr].t) & tmask;
        rbits[rr] = flag_bits<K, VEC>(f[rr].r) & rmask;
      }
    }
  };

  auto issue_dense = [&](const Cursor& c, RowData<Est, K> (&dd)[R]) __attribute__((always_inline)) {
    const TilePos q = tile_pos(c);
    const ItemRows<R> ir = item_rows(c);
    const int64_t eb = ir.wb * T;  // element index of the base row
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      RowData<Est, K>& d = dd[rr];
      const uint32_t off = ir.roff[rr] + q.cs;
      const uint32_t last = ir.roff[rr] + T32 - 1;
      load_s<S, K, VEC>(p.r, eb, off, last, d.s[0]);
      if constexpr (NS >= 2) load_s<S, K, VEC>(p.v, eb, off, last, d.s[1]);
      if constexpr (NS >= 3) load_s<S, K, VEC>(p.aux, eb, off, last, d.s[2]);
      if constexpr (NS >= 5) {
        load_s<S, K, VEC>(p.pi, eb, off, last, d.s[3]);
        load_s<S, K, VEC>(p.mu, eb, off, last, d.s[4]);
      }
      // the team-first lane's scan predecessor: one address per team part (one request)
      const uint32_t noff = ir.roff[rr] + q.tn;
      if constexpr (Tr::kRetrace) {
        d.nb[0] = load1<S>(p.aux, eb, noff);
        d.nb[1] = load1<S>(p.pi, eb, noff);
        d.nb[2] = load1<S>(p.mu, eb, noff);
      } else if constexpr (Tr::kNbValue) {
        d.nb[0] = load1<S>(p.v, eb, noff);
      } else if constexpr (Tr::kNbDone && USE_FLAGS) {
        d.nbf[0] = __builtin_nontemporal_load(at(p.term + eb, noff));
        d.nbf[1] = __builtin_nontemporal_load(at(p.trunc + eb, noff));
      }
      d.rowv = load1<S>(p.row, ir.wb, ir.rsel[rr]);
    }
  };

  // Truncation bootstraps of each lane's chunk; lanes without a truncated step
  // read the array's first chunk instead (one line shared by all waves).
  auto issue_gather = [&](const Cursor& c, const unsigned (&tbits)[R], const unsigned (&rbits)[R],
                          RowData<Est, K> (&dd)[R]) __attribute__((always_inline)) {
    if constexpr (GATHER_TB) {
      const TilePos q = tile_pos(c);
      const ItemRows<R> ir = item_rows(c);
      const int64_t eb = ir.wb * T;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        RowData<Est, K>& d = dd[rr];
        const uint32_t off = ir.roff[rr] + q.cs;
        const uint32_t last = ir.roff[rr] + T32 - 1;
        const unsigned need = rbits[rr] & ~tbits[rr];
        if constexpr (VEC) {
          load_s<S, K, true>(p.tboot, need ? eb : 0, need ? off : 0u, 0u, d.tb);
        } else {
#pragma unroll
          for (int m = 0; m < K; ++m) {
            const uint32_t col = off + m < last ? off + m : last;
            const bool sel = (need >> m) & 1u;
            d.tb[m] = load1<S>(p.tboot, sel ? eb : 0, sel ? col : 0u);
          }
        }
      }
    }
  };

  auto issue_data = [&](const Cursor& c, const unsigned (&tbits)[R], const unsigned (&rbits)[R],
                        RowData<Est, K> (&dd)[R]) __attribute__((always_inline)) {
    issue_dense(c, dd);
    issue_gather(c, tbits, rbits, dd);
  };

  const ScanScalars sc{gamma, lam, gl, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0, p.has_tboot != 0};

  // Scan one row of an item and form its outputs; C is the running value of the row.
  auto scan_row = [&](int64_t k, int rr, const TilePos& q, bool row_ok, const RowData<Est, K>& d,
                      unsigned tbits, unsigned rbits, double& C, float (&o0)[K], float (&o1)[K])
      __attribute__((always_inline)) {
    if (q.first) {
      if constexpr (Tr::kBackwardRl) C = 0.0;
      else C = (row_ok && p.has_row) ? (double)d.rowv : 0.0;
    }
    const int nv = row_ok ? q.nv : 0;

    // the team-first lane's scan predecessor, reloaded from memory
    PredIn pred{0.0f, 0.0, 0u};
    if constexpr (Tr::kRetrace) {
      pred.v = d.nb[0];
      if constexpr (!__is_same(S, F32S)) {
        pred.c = q.nb_ok ? retrace_c_fast(lam, d.nb[1], d.nb[2]) : 0.0;
      } else {
        const double ratio = (double)d.nb[1] / (double)d.nb[2];
        pred.c = q.nb_ok ? lam * (ratio < 1.0 ? ratio : 1.0) : 0.0;
      }
    } else if constexpr (Tr::kNbValue) {
      pred.v = d.nb[0];
    } else if constexpr (Tr::kNbDone && USE_FLAGS) {
      const unsigned dn = ((unsigned)(d.nbf[0] != 0) & tmask) | ((unsigned)(d.nbf[1] != 0) & rmask);
      pred.done = (q.nb_ok && dn) ? 1u : 0u;
    }
    const LanePairs<K> lp = build_pairs<Est, K, VEC, !__is_same(S, F32S)>(d, sc, tbits, rbits, q.cs, T, nv, team_first_lane, pred);

    // ---- (a3) serial fold, (a4) wave scan over lanes
    const AB incl = lane_scan<(W > 1 ? 64 : L)>(fold_lane<K>(lp.e));

    // ---- (a5) block carry across the waves of a team (LDS)
    double Cw = C;        // value entering this wave's innermost step
    double C_next = 0.0;  // value leaving the tile
    if constexpr (W > 1) {
      const int buf = (int)(k & 1);
      if (lane == 63) {
        s_tot[buf][team][rr][w][0] = incl.a;
        s_tot[buf][team][rr][w][1] = incl.b;
      }
      __syncthreads();
      double x = C;
#pragma unroll
      for (int u = 0; u < W; ++u) {
        if (u == w) Cw = x;
        x = __builtin_fma(s_tot[buf][team][rr][u][0], x, s_tot[buf][team][rr][u][1]);
      }
      C_next = x;
    }

    // ---- (a6) value entering each lane, then re-walk; (a7) epilogue
    const double y_last = __builtin_fma(incl.a, Cw, incl.b);  // value after this lane's steps
    const double from_below = shift_up_f64(y_last);
    const double x_in = team_first_lane ? Cw : from_below;
    if constexpr (W == 1) C_next = group_last_f64<L>(y_last, lane);
    double xs[K];
    rewalk<K>(lp.e, x_in, xs);
    epilogue<Est, K>(d, lp, sc, x_in, xs, o0, o1);
    C = C_next;
  };

  // Scan all rows of item k, then store them (stores last: a pending store
  // makes the next wait on a load drain the memory counter).
  auto compute = [&](int64_t k, const Cursor& c, const RowData<Est, K> (&dd)[R], const unsigned (&tbits)[R],
                     const unsigned (&rbits)[R], double (&C)[R]) __attribute__((always_inline)) {
    const TilePos q = tile_pos(c);
    const ItemRows<R> ir = item_rows(c);
    float o0[R][K], o1[R][K];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) scan_row(k, rr, q, ir.ok[rr], dd[rr], tbits[rr], rbits[rr], C[rr], o0[rr], o1[rr]);
    const int64_t eb = ir.wb * T;
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int nv = ir.ok[rr] ? q.nv : 0;
      if (nv > 0) {
        const uint32_t off = ir.roff[rr] + q.cs;
        store_s<S, K, VEC>(p.out0, eb, off, nv, o0[rr]);
        if constexpr (OUT1) store_s<S, K, VEC>(p.out1, eb, off, nv, o1[rr]);
      }
    }
  };

  // ---------------------------------------------------------------- one item per team
  // The grid holds a team for every row group, so a team scans the tiles of
  // one row group and exits; the hardware refills its slot with a new block.
  // Flags and inputs go out together, the bootstrap gather as soon as the
  // flags land, and nothing is fetched for a later item.
  if constexpr (ONE) {
    double C[R];
#pragma unroll
    for (int rr = 0; rr < R; ++rr) C[rr] = 0.0;
    Cursor c{0, 0, 0};
    for (int64_t ts = 0; ts < ntiles; ++ts) {
      FlagRaw<K> F[R];
      RowData<Est, K> D[R];
      unsigned bt[R], br[R];
      issue_flags(c, F);
      issue_dense(c, D);
      decode(F, bt, br);
      issue_gather(c, bt, br, D);
      compute(c.k, c, D, bt, br, C);
      c = advance(c);
    }
    return;
  }

  // ---------------------------------------------------------------- the pipeline
  // Two register sets (X: even items, Y: odd items) swap roles each step, so no
  // in-flight load is ever copied.  Step k: decode the flags of item k+1, issue
  // the flags of item k+2 and the inputs + bootstrap gather of item k+1, then
  // scan and store item k.
  FlagRaw<K> FX[R], FY[R];
  RowData<Est, K> DX[R], DY[R];
  Cursor c0{0, 0, 0};
  Cursor c1 = advance(c0);
  Cursor c2 = advance(c1);
  unsigned bt_cur[R], br_cur[R], bt_nxt[R], br_nxt[R];
  issue_flags(c0, FX);
  issue_flags(c1, FY);
  decode(FX, bt_cur, br_cur);
  issue_data(c0, bt_cur, br_cur, DX);
  double C[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) C[rr] = 0.0;
  for (int64_t k = 0; k < n_items; k += 2) {
    // item k (set X)
    decode(FY, bt_nxt, br_nxt);
    issue_flags(c2, FX);
    issue_data(c1, bt_nxt, br_nxt, DY);
    compute(k, c0, DX, bt_cur, br_cur, C);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      bt_cur[rr] = bt_nxt[rr];
      br_cur[rr] = br_nxt[rr];
    }
    c0 = c1;
    c1 = c2;
    c2 = advance(c2);
    // item k+1 (set Y)
    decode(FX, bt_nxt, br_nxt);
    issue_flags(c2, FY);
    issue_data(c1, bt_nxt, br_nxt, DX);
    compute(k + 1, c0, DY, bt_cur, br_cur, C);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      bt_cur[rr] = bt_nxt[rr];
      br_cur[rr] = br_nxt[rr];
    }
    c0 = c1;
    c1 = c2;
    c2 = advance(c2);
  }
}

}  // namespace rlscan
