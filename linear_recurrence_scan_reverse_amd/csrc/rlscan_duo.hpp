// rlscan_duo.hpp -- the item kernels: rows of 64 to 512 steps, cut into items
// of 1 KiB of every array (256 float32 or 512 16-bit elements; a variant of
// 512 bytes for 16-bit rows of 64-256 steps), each item G = 64 / L whole rows
// of L lanes.  A wave scans several items:
//  * duo_kernel (float32): two items, the second with up to NLMAX of its input
//    streams staged in the wave's own LDS slot by DMA;
//  * duo_reg_kernel: two items, both held in registers as raw bytes;
//  * multi_reg_kernel: four items in registers as a software pipeline.
//
// A kernel that gives each wave one item (the pipelined kernel's one-item
// form) requests every item of a CU at once, so the waves reach their compute
// together at the end of the load phase and the compute is exposed.  With
// several items per wave a wave can scan one item while the next ones land.
// gfx9 counts a wave's loads with one in-order counter, so the order in which
// items and their flag-dependent bootstrap gathers are requested decides what
// each wait covers; each kernel states its order below.  The per-lane scan
// code is the one every kernel of the library shares (stream_tile: pairs,
// fold, lane scan, re-walk, epilogue).
#pragma once

#include "rlscan_stream.hpp"

namespace rlscan {

constexpr int kDuoItemBytes = 1024;  // bytes of every array in one item

// Four float32 values at an LDS byte address (16-byte aligned).
__device__ __forceinline__ void lds_read4f(const char* q, float (&o)[4]) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(q);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}

// ----------------------------------------------------------------- two items, the second through LDS
// Order inside a wave (the bootstrap gather of each item is issued as soon
// as its flags are known):
//   1. item A: flags, input streams, row value -> registers;
//   2. item B: NL input streams -> LDS (DMA), the rest, flags, row value -> registers;
//   3. A's flags decoded, A's truncation bootstraps gathered;
//   4. wait for everything; B's flags decoded, B's bootstraps gathered;
//   5. A scanned and stored (B's gather in flight);
//   6. B read from LDS, scanned and stored.
// A wave that mixes LDS DMA with ordinary loads gets no finer waits from the
// compiler than "everything" (its counter tracking takes the two kinds as
// unordered), so A is scanned once B has landed too.  The LDS slot costs no
// registers, so occupancy stays that of a one-item kernel.
//
// Template parameters: estimator tag (not the two-output pass), team width L
// (T == 4 L), OPT (bit 0 flags, bit 1 second output), storage format S
// (float32 only), NLMAX.  Every dense array 16-byte aligned, flag arrays
// 4-byte aligned (checked by the launcher).  Blocks of 4 waves take items
// 8 b + w and 8 b + 4 + w.
// Retrace forms its trace quotient pi / mu from the fp32 reciprocal of mu
// refined by one fp64 Newton step (retrace_c_fast, relative error about
// 1e-14) instead of an fp64 division: this kernel computes two items per wave
// after both have landed, so its vector instructions count.  Measured at
// 16384 x 256 on one MI355X: 20.0 -> 19.75 us (the one-item form measured
// slower with it and keeps the division).  The register forms do the same,
// and in 16-bit storage they also take the fast exp of V-trace, as every
// kernel does for those formats.
template <class Est, int L, int OPT, class S = F32S, int NLMAX = 3>
__global__ void __launch_bounds__(256) duo_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr int ES = (int)sizeof(typename S::T);  // bytes per stored value
  constexpr int K = 16 / ES;                      // steps per lane
  constexpr int ITEM = kDuoItemBytes / ES;        // elements per item
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  constexpr bool FAST = Tr::kRetrace;
  constexpr int G = 64 / L;   // rows per item
  constexpr int SPAN = L * K;  // row length
  static_assert(__is_same(S, F32S), "float32 storage (16-bit rows take the register forms)");
  static_assert(!Tr::kDual, "one recurrence per pass");
  static_assert(G * SPAN == ITEM, "an item is whole rows");

  // B's first NL streams go through LDS (at most NLMAX, 1 KiB each per wave:
  // three take 12 KiB per block, so eight blocks fit a CU's LDS with room to
  // spare); the rest -> registers
  constexpr int NL = NS < NLMAX ? NS : NLMAX;
  __shared__ __attribute__((aligned(16))) char s_b[4][NL][kDuoItemBytes];  // each wave's second item, memory order

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int team = lane / L;  // row of the item
  const int g = lane & (L - 1);
  const bool team_first_lane = g == 0;
  const uint32_t cs = REV ? (uint32_t)(SPAN - (g + 1) * K) : (uint32_t)(g * K);  // column of the lane's chunk
  const uint32_t lds_off = (uint32_t)((team * SPAN + (int)cs) * ES);             // its byte offset in the item
  const int64_t E = p.E, T = p.T;
  const int64_t items = (E + G - 1) / G;
  const int64_t item_a = (int64_t)blockIdx.x * 8 + w;
  const int64_t item_b = item_a + 4;
  if (item_a >= items) return;  // (wave-uniform; the kernel has no block barrier)
  const bool has_b = item_b < items;
  const int64_t item_bc = has_b ? item_b : item_a;  // a valid item for the loads

  const double gamma = p.gamma, lam = p.lam;
  const ScanScalars sc{gamma, lam, gamma * lam, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0, p.has_tboot != 0};
  const unsigned tmask = p.has_term ? ~0u : 0u;
  const unsigned rmask = p.has_trunc ? ~0u : 0u;
  const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};

  // rows of this lane in items A and B (clamped into the array for the loads)
  const int64_t row_a = item_a * G + team, row_b = item_bc * G + team;
  const bool ok_a = row_a < E, ok_b = has_b && row_b < E;
  const int64_t ra = ok_a ? row_a : E - 1, rb = row_b < E ? row_b : E - 1;

  // ---- 1. item A -> registers
  LaneIn<Est, K> da;
  unsigned fta[K], fra[K];
#pragma unroll
  for (int st = 0; st < NS; ++st) load_s<S, K, true>(srcs[st], ra * T, cs, 0u, da.s[st]);
  if constexpr (USE_FLAGS) {
    load_flag_raw<K, true>(p.term + ra * T, cs, 0u, fta);
    load_flag_raw<K, true>(p.trunc + ra * T, cs, 0u, fra);
  }
  da.rowv = load1<S>(p.row, ra, 0u);

  // ---- 2. item B: streams -> LDS (lane l moves bytes 16 l .. 16 l + 15 of
  // the item, clamped into the array), flags and row value -> registers
  {
    int64_t bo = item_bc * kDuoItemBytes + 16 * lane;
    if (bo > E * T * ES - 16) bo = E * T * ES - 16;
#pragma unroll
    for (int st = 0; st < NL; ++st)
      __builtin_amdgcn_global_load_lds((gbl_void_ptr)(reinterpret_cast<const char*>(srcs[st]) + bo),
                                       (lds_void_ptr)&s_b[w][st][0], 16, 0, 0);
  }
  LaneIn<Est, K> db;
#pragma unroll
  for (int st = NL; st < NS; ++st) load_s<S, K, true>(srcs[st], rb * T, cs, 0u, db.s[st]);
  unsigned ftb[K], frb[K];
  if constexpr (USE_FLAGS) {
    load_flag_raw<K, true>(p.term + rb * T, cs, 0u, ftb);
    load_flag_raw<K, true>(p.trunc + rb * T, cs, 0u, frb);
  }
  db.rowv = load1<S>(p.row, rb, 0u);

  // ---- 3. A's flags and bootstrap gather
  unsigned tba = 0, rba = 0, tbb = 0, rbb = 0;
#pragma unroll
  for (int m = 0; m < K; ++m) da.tb[m] = db.tb[m] = 0.0f;
  if constexpr (USE_FLAGS) {
    tba = flag_bits<K, true>(fta) & tmask;
    rba = flag_bits<K, true>(fra) & rmask;
  }
  if constexpr (GATHER_TB) {
    if ((rba & ~tba) != 0u && p.has_tboot) load_s<S, K, true>(p.tboot, ra * T, cs, 0u, da.tb);
  }

  // ---- 4. everything landed (B's DMA included); B's flags and gather
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  if constexpr (USE_FLAGS) {
    tbb = flag_bits<K, true>(ftb) & tmask;
    rbb = flag_bits<K, true>(frb) & rmask;
  }
  if constexpr (GATHER_TB) {
    if ((rbb & ~tbb) != 0u && p.has_tboot) load_s<S, K, true>(p.tboot, rb * T, cs, 0u, db.tb);
  }

  // ---- 5. item A
  {
    double C = 0.0;
    if constexpr (!Tr::kBackwardRl) C = (ok_a && p.has_row) ? (double)da.rowv : 0.0;
    PredIn carry{0.0f, 0.0, 0u};  // a row is one tile: no scan predecessor
    float o0[K], o1[K];
    stream_tile<Est, L, K, false, FAST>(da, sc, tba, rba, cs, T, team_first_lane, lane, C, carry, o0, o1);
    if (G == 1 || ok_a) {
      store_s<S, K, true>(p.out0, ra * T, cs, K, o0);
      if constexpr (OUT1) store_s<S, K, true>(p.out1, ra * T, cs, K, o1);
    }
  }

  // ---- 6. item B
  if (!has_b) return;
#pragma unroll
  for (int st = 0; st < NL; ++st) lds_read4f(&s_b[w][st][lds_off], db.s[st]);
  {
    double C = 0.0;
    if constexpr (!Tr::kBackwardRl) C = (ok_b && p.has_row) ? (double)db.rowv : 0.0;
    PredIn carry{0.0f, 0.0, 0u};
    float o0[K], o1[K];
    stream_tile<Est, L, K, false, FAST>(db, sc, tbb, rbb, cs, T, team_first_lane, lane, C, carry, o0, o1);
    if (G == 1 || ok_b) {
      store_s<S, K, true>(p.out0, rb * T, cs, K, o0);
      if constexpr (OUT1) store_s<S, K, true>(p.out1, rb * T, cs, K, o1);
    }
  }
}

// ----------------------------------------------------------------- both items in registers
// The same two items per wave with item B held in registers too, as the raw
// bytes of each stream and lane (converted only when B is scanned), so no LDS
// DMA mixes with the ordinary loads and the compiler's waits stay exact: A is
// scanned as soon as its own loads have landed, while B's are still in
// flight.  In the LDS form every wave waits for both items, so the waves of a
// CU, whose requests all went out at once, mostly start computing together at
// the end of the load phase; here half of that work moves into it.  Measured
// at 16384 x 256 on one MI355X: bfloat16 discounted returns 9.1 -> 7.9 us,
// V-trace 14.1 -> 12.2 us against the LDS form; float32 discounted returns
// 10.3 -> 9.4 us, Retrace 19.5 -> 20.1 us (Retrace keeps the LDS form there).  Request order: A's flags, A's streams, B's flags, A's bootstraps
// (once A's flags are in), B's streams, B's bootstraps (once B's flags are
// in); then A is scanned and stored, then B.  Bootstraps and stores go
// through buffer resources over the item (lanes without a bootstrap to fetch,
// and rows past E, fall outside the resource and touch no memory), so no
// branch surrounds a request.
constexpr uint32_t kDuoOff = 0x80000000u;  // past every item resource

template <class S, int IB = kDuoItemBytes>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t duo_item_rs(const void* base, int64_t item, int64_t total_bytes) {
  const int64_t b0 = item * IB;
  const int64_t n = total_bytes - b0 < IB ? total_bytes - b0 : IB;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + b0, 0, (int)n,
                                           0x00020000);
}

// A lane's raw bytes of one array in one item: 16 (u32x4) or 8 (u32x2).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int LB> struct RawOf;
template <> struct RawOf<16> { typedef u32x4 T; };
template <> struct RawOf<8> { typedef u32x2 T; };

template <int LB>
__device__ __forceinline__ typename RawOf<LB>::T raw_buffer_load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (LB == 16) return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2);
  else return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 2);
}
template <int LB>
__device__ __forceinline__ void raw_buffer_store(typename RawOf<LB>::T v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (LB == 16) __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 2);
  else __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, 2);
}
// K values of format S from 8 raw bytes (16-bit formats, K = 4).
template <class S, int K>
__device__ __forceinline__ void unpack8(const u32x2 v, float (&o)[K]) {
  static_assert(!__is_same(S, F32S) && K == 4, "four 16-bit values");
  o[0] = s_to_f32<S>((uint16_t)v.x);
  o[1] = s_to_f32<S>((uint16_t)(v.x >> 16));
  o[2] = s_to_f32<S>((uint16_t)v.y);
  o[3] = s_to_f32<S>((uint16_t)(v.y >> 16));
}
template <class S, int K>
__device__ __forceinline__ u32x2 pack8(const float (&o)[K]) {
  static_assert(!__is_same(S, F32S) && K == 4, "four 16-bit values");
  u32x2 q;
  q.x = (uint32_t)f32_to_s<S>(o[0]) | ((uint32_t)f32_to_s<S>(o[1]) << 16);
  q.y = (uint32_t)f32_to_s<S>(o[2]) | ((uint32_t)f32_to_s<S>(o[3]) << 16);
  return q;
}

// K values of format S from 16 raw bytes.
template <class S, int K>
__device__ __forceinline__ void unpack16(const u32x4 v, float (&o)[K]) {
  if constexpr (__is_same(S, F32S)) {
    static_assert(K == 4, "four float32 values");
    const f32x4 f = __builtin_bit_cast(f32x4, v);
    o[0] = f.x; o[1] = f.y; o[2] = f.z; o[3] = f.w;
  } else {
    static_assert(K == 8, "eight 16-bit values");
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = s_to_f32<S>((uint16_t)w[i]);
      o[2 * i + 1] = s_to_f32<S>((uint16_t)(w[i] >> 16));
    }
  }
}
// K values of format S packed into 16 bytes.
template <class S, int K>
__device__ __forceinline__ u32x4 pack16(const float (&o)[K]) {
  if constexpr (__is_same(S, F32S)) {
    return __builtin_bit_cast(u32x4, f32x4{o[0], o[1], o[2], o[3]});
  } else {
    u32x4 q;
    q.x = (uint32_t)f32_to_s<S>(o[0]) | ((uint32_t)f32_to_s<S>(o[1]) << 16);
    q.y = (uint32_t)f32_to_s<S>(o[2]) | ((uint32_t)f32_to_s<S>(o[3]) << 16);
    q.z = (uint32_t)f32_to_s<S>(o[4]) | ((uint32_t)f32_to_s<S>(o[5]) << 16);
    q.w = (uint32_t)f32_to_s<S>(o[6]) | ((uint32_t)f32_to_s<S>(o[7]) << 16);
    return q;
  }
}

template <class Est, int L, int OPT, class S = F32S, int LB = 16>
__global__ void __launch_bounds__(256) duo_reg_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  using RawT = typename RawOf<LB>::T;
  constexpr int ES = (int)sizeof(typename S::T);
  constexpr int K = LB / ES;     // steps per lane
  constexpr int IB = 64 * LB;    // bytes of every array in one item
  constexpr int ITEM = IB / ES;  // elements per item
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  constexpr bool FAST = Tr::kRetrace || !__is_same(S, F32S);
  constexpr int G = 64 / L;
  constexpr int SPAN = L * K;
  static_assert(!Tr::kDual, "one recurrence per pass");
  static_assert(G * SPAN == ITEM, "an item is whole rows");

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int team = lane / L;
  const int g = lane & (L - 1);
  const bool team_first_lane = g == 0;
  const uint32_t cs = REV ? (uint32_t)(SPAN - (g + 1) * K) : (uint32_t)(g * K);
  const uint32_t boff = (uint32_t)((team * SPAN + (int)cs) * ES);  // lane's byte offset in its item
  const int64_t E = p.E, T = p.T;
  const int64_t total = E * T * ES;
  const int64_t items = (E + G - 1) / G;
  const int64_t item_a = (int64_t)blockIdx.x * 8 + w;
  const int64_t item_b = item_a + 4;
  if (item_a >= items) return;  // (wave-uniform; the kernel has no block barrier)
  const bool has_b = item_b < items;
  const int64_t item_bc = has_b ? item_b : item_a;

  const double gamma = p.gamma, lam = p.lam;
  const ScanScalars sc{gamma, lam, gamma * lam, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0, p.has_tboot != 0};
  const unsigned tmask = p.has_term ? ~0u : 0u;
  const unsigned rmask = p.has_trunc ? ~0u : 0u;
  const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};

  const int64_t row_a = item_a * G + team, row_b = item_bc * G + team;
  const bool ok_a = row_a < E, ok_b = has_b && row_b < E;
  const int64_t ra = ok_a ? row_a : E - 1, rb = row_b < E ? row_b : E - 1;
  auto raw_at = [&](const float* base, int64_t row) -> RawT {
    return __builtin_nontemporal_load(
        reinterpret_cast<const RawT*>(reinterpret_cast<const char*>(base) + (row * T + cs) * ES));
  };
  auto unpack = [&](const RawT v, float (&o)[K]) {
    if constexpr (LB == 16) unpack16<S, K>(v, o);
    else unpack8<S, K>(v, o);
  };
  auto pack = [&](const float (&o)[K]) -> RawT {
    if constexpr (LB == 16) return pack16<S, K>(o);
    else return pack8<S, K>(o);
  };

  // A's flags and streams, B's flags
  unsigned fta[K], fra[K], ftb[K], frb[K];
  if constexpr (USE_FLAGS) {
    load_flag_raw<K, true>(p.term + ra * T, cs, 0u, fta);
    load_flag_raw<K, true>(p.trunc + ra * T, cs, 0u, fra);
  }
  const float rowa = load1<S>(p.row, ra, 0u);
  RawT xa[NS], xb[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) xa[st] = raw_at(srcs[st], ra);
  if constexpr (USE_FLAGS) {
    load_flag_raw<K, true>(p.term + rb * T, cs, 0u, ftb);
    load_flag_raw<K, true>(p.trunc + rb * T, cs, 0u, frb);
  }
  const float rowb = load1<S>(p.row, rb, 0u);
  asm volatile("" ::: "memory");

  // A's bootstraps (waits for A's flags only; the empty asm takes A's flag
  // words here, so their decode cannot move above B's requests)
  unsigned tba = 0, rba = 0, tbb = 0, rbb = 0;
  if constexpr (USE_FLAGS) {
#pragma unroll
    for (int i = 0; i < K / 4; ++i) asm volatile("" : "+v"(fta[i]), "+v"(fra[i])::"memory");
    tba = flag_bits<K, true>(fta) & tmask;
    rba = flag_bits<K, true>(fra) & rmask;
  }
  RawT ga = RawT(0u), gb = RawT(0u);
  if constexpr (GATHER_TB) {
    const bool need = ok_a && (rba & ~tba) != 0u && p.has_tboot;
    ga = raw_buffer_load<LB>(duo_item_rs<S, IB>(p.tboot, item_a, total), need ? boff : kDuoOff);
  }
  // B's streams, then B's bootstraps (waits for B's flags only).  The empty
  // asm takes B's flag words after B's streams are requested, so the compiler
  // cannot decode them (and wait for them, and so for A's streams) earlier.
#pragma unroll
  for (int st = 0; st < NS; ++st) xb[st] = raw_at(srcs[st], rb);
  if constexpr (USE_FLAGS) {
#pragma unroll
    for (int i = 0; i < K / 4; ++i) asm volatile("" : "+v"(ftb[i]), "+v"(frb[i])::"memory");
  }
  if constexpr (USE_FLAGS) {
    tbb = flag_bits<K, true>(ftb) & tmask;
    rbb = flag_bits<K, true>(frb) & rmask;
  }
  if constexpr (GATHER_TB) {
    const bool need = ok_b && (rbb & ~tbb) != 0u && p.has_tboot;
    gb = raw_buffer_load<LB>(duo_item_rs<S, IB>(p.tboot, item_bc, total), need ? boff : kDuoOff);
  }

  // one item: unpack, scan, store (rows past E fall outside the output resource)
  auto item = [&](int64_t it, const RawT (&x)[NS], const RawT gt, float rowv, unsigned tbits, unsigned rbits,
                  bool ok) {
    LaneIn<Est, K> d;
#pragma unroll
    for (int st = 0; st < NS; ++st) unpack(x[st], d.s[st]);
    unpack(gt, d.tb);
    d.rowv = rowv;
    double C = 0.0;
    if constexpr (!Tr::kBackwardRl) C = (ok && p.has_row) ? (double)rowv : 0.0;
    PredIn carry{0.0f, 0.0, 0u};
    float o0[K], o1[K];
    stream_tile<Est, L, K, false, FAST>(d, sc, tbits, rbits, cs, T, team_first_lane, lane, C, carry, o0, o1);
    raw_buffer_store<LB>(pack(o0), duo_item_rs<S, IB>(p.out0, it, total), boff);
    if constexpr (OUT1) raw_buffer_store<LB>(pack(o1), duo_item_rs<S, IB>(p.out1, it, total), boff);
  };
  item(item_a, xa, ga, rowa, tba, rba, ok_a);
  if (!has_b) return;
  item(item_b, xb, gb, rowb, tbb, rbb, ok_b);
}

// ----------------------------------------------------------------- NI items per wave, in registers
// Wave w of block b scans items b * 4 NI + 4 i + w, i = 0 .. NI - 1, as a
// software pipeline: while item i is scanned, the streams of items i + 1 and
// i + 2, the bootstraps of item i + 1 and the flags of i + 2 and i + 3 are in
// flight.  Per iteration i the wave requests bootstraps(i + 1) (its flags
// landed with the streams of item i, which were requested before them),
// streams(i + 2) and flags(i + 3), then scans and stores item i; the only
// waits are for what item i uses.  Items past the last are scanned on a
// clamped item's data and not stored (their store offset falls outside the
// output resource), so no branch surrounds a request.
template <class Est, int L, int OPT, class S, int NI>
__global__ void __launch_bounds__(256) multi_reg_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr int ES = (int)sizeof(typename S::T);
  constexpr int K = 16 / ES;
  constexpr int ITEM = kDuoItemBytes / ES;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  constexpr bool FAST = Tr::kRetrace || !__is_same(S, F32S);
  constexpr int G = 64 / L;
  constexpr int SPAN = L * K;
  static_assert(!Tr::kDual, "one recurrence per pass");
  static_assert(G * SPAN == ITEM, "an item is whole rows");
  static_assert(NI >= 2 && NI <= 4, "items per wave");

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int team = lane / L;
  const int g = lane & (L - 1);
  const bool team_first_lane = g == 0;
  const uint32_t cs = REV ? (uint32_t)(SPAN - (g + 1) * K) : (uint32_t)(g * K);
  const uint32_t boff = (uint32_t)((team * SPAN + (int)cs) * ES);
  const int64_t E = p.E, T = p.T;
  const int64_t total = E * T * ES;
  const int64_t items = (E + G - 1) / G;
  const int64_t first = (int64_t)blockIdx.x * (4 * NI) + w;
  if (first >= items) return;  // (wave-uniform; the kernel has no block barrier)

  const double gamma = p.gamma, lam = p.lam;
  const ScanScalars sc{gamma, lam, gamma * lam, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0, p.has_tboot != 0};
  const unsigned tmask = p.has_term ? ~0u : 0u;
  const unsigned rmask = p.has_trunc ? ~0u : 0u;
  const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};

  int64_t it[NI], rr[NI];
  bool ok[NI], has[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t t = first + 4 * i;
    has[i] = t < items;
    it[i] = has[i] ? t : first;  // a valid item for the requests
    const int64_t row = it[i] * G + team;
    ok[i] = has[i] && row < E;
    rr[i] = row < E ? row : E - 1;
  }
  unsigned ft[NI][K], fr[NI][K];
  float rowv[NI];
  u32x4 x[NI][NS], gt[NI];
  unsigned tb[NI], rb[NI];

  auto req_flags = [&](int i) {
    if constexpr (USE_FLAGS) {
      load_flag_raw<K, true>(p.term + rr[i] * T, cs, 0u, ft[i]);
      load_flag_raw<K, true>(p.trunc + rr[i] * T, cs, 0u, fr[i]);
    }
    rowv[i] = load1<S>(p.row, rr[i], 0u);
  };
  auto req_streams = [&](int i) {
#pragma unroll
    for (int st = 0; st < NS; ++st)
      x[i][st] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(srcs[st]) + (rr[i] * T + cs) * ES));
  };
  // decode item i's flags (the empty asm pins the wait for them here) and
  // request its bootstraps
  auto req_gather = [&](int i) {
    tb[i] = rb[i] = 0u;
    if constexpr (USE_FLAGS) {
#pragma unroll
      for (int j = 0; j < K / 4; ++j) asm volatile("" : "+v"(ft[i][j]), "+v"(fr[i][j])::"memory");
      tb[i] = flag_bits<K, true>(ft[i]) & tmask;
      rb[i] = flag_bits<K, true>(fr[i]) & rmask;
    }
    gt[i] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (GATHER_TB) {
      const bool need = ok[i] && (rb[i] & ~tb[i]) != 0u && p.has_tboot;
      gt[i] = __builtin_amdgcn_raw_buffer_load_b128(duo_item_rs<S>(p.tboot, it[i], total), need ? boff : kDuoOff,
                                                    0, 2);
    }
  };
  auto scan_item = [&](int i) {
    LaneIn<Est, K> d;
#pragma unroll
    for (int st = 0; st < NS; ++st) unpack16<S, K>(x[i][st], d.s[st]);
    unpack16<S, K>(gt[i], d.tb);
    d.rowv = rowv[i];
    double C = 0.0;
    if constexpr (!Tr::kBackwardRl) C = (ok[i] && p.has_row) ? (double)rowv[i] : 0.0;
    PredIn carry{0.0f, 0.0, 0u};
    float o0[K], o1[K];
    stream_tile<Est, L, K, false, FAST>(d, sc, tb[i], rb[i], cs, T, team_first_lane, lane, C, carry, o0, o1);
    const uint32_t so = has[i] ? boff : kDuoOff;
    __builtin_amdgcn_raw_buffer_store_b128(pack16<S, K>(o0), duo_item_rs<S>(p.out0, it[i], total), so, 0, 2);
    if constexpr (OUT1)
      __builtin_amdgcn_raw_buffer_store_b128(pack16<S, K>(o1), duo_item_rs<S>(p.out1, it[i], total), so, 0, 2);
  };

  // prologue: flags and streams of items 0 and 1, flags of item 2, then the
  // bootstraps of item 0
  // (each empty asm keeps the compiler from reordering requests across it)
  req_flags(0);
  asm volatile("" ::: "memory");
  req_streams(0);
  asm volatile("" ::: "memory");
  req_flags(1);
  asm volatile("" ::: "memory");
  req_streams(1);
  asm volatile("" ::: "memory");
  if constexpr (NI > 2) req_flags(2);
  asm volatile("" ::: "memory");
  req_gather(0);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    asm volatile("" ::: "memory");
    if (i + 1 < NI) req_gather(i + 1);
    asm volatile("" ::: "memory");
    if (i + 2 < NI) req_streams(i + 2);
    asm volatile("" ::: "memory");
    if (i + 3 < NI) req_flags(i + 3);
    asm volatile("" ::: "memory");
    scan_item(i);
  }
}

}  // namespace rlscan
