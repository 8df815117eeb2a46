// rlscan_duo.hpp -- rows of 64, 128 or 256 steps (one 256-element item of
// every [E,T] array holds G = 64 / L whole rows): each wave scans two items,
// the first loaded into registers and the second into LDS by DMA, both
// requested before either is scanned.
//
// A kernel that gives each wave one item (the pipelined kernel's one-item
// form) holds its inputs in registers; at full occupancy a CU then has 32
// items in flight, and the rows the first round of waves does not cover wait
// for slots to free before their loads start.  A plain streaming kernel moving
// the same arrays ran fastest with two items per wave (every item requested at
// once).  Here the second item costs few registers: up to three of its input
// streams land in the wave's own LDS slot (1 KiB per stream and wave; 12 KiB
// per block at most, so eight blocks fit a CU) and the rest in registers, so
// occupancy stays that of the one-item kernel while twice the bytes are
// requested.  The per-lane
// scan code is the one every kernel of the library shares (stream_tile:
// pairs, fold, lane scan, re-walk, epilogue).
//
// Order inside a wave (the flag-dependent bootstrap gather of each item is
// issued as soon as its flags are known):
//   1. item A: flags, input streams, row value -> registers;
//   2. item B: input streams -> LDS (DMA), flags and row value -> registers;
//   3. A's flags decoded, A's truncation bootstraps gathered;
//   4. wait for everything; B's flags decoded, B's bootstraps gathered;
//   5. A scanned and stored (B's gather in flight);
//   6. B read from LDS, scanned and stored.
// A wave that mixes LDS DMA with ordinary loads gets no finer waits from the
// compiler than "everything" (its counter tracking takes the two kinds as
// unordered), so A is scanned once B has landed too: every item of the wave
// is requested at once, as in the plain streaming kernel the design follows.
#pragma once

#include "rlscan_stream.hpp"

namespace rlscan {

constexpr int kDuoItem = 256;  // elements of every array in one item

// Template parameters: estimator tag (not the two-output pass), team width L
// (T == 4 L), OPT (bit 0 flags, bit 1 second output).  Float32 storage; every
// dense array 16-byte aligned, flag arrays 4-byte aligned (checked by the
// launcher).  Blocks of 4 waves take items 8 b + w and 8 b + 4 + w.
// Retrace forms its trace quotient pi / mu from the fp32 reciprocal of mu
// refined by one fp64 Newton step (retrace_c_fast, relative error about
// 1e-14) instead of an fp64 division: this kernel computes two items per wave
// after both have landed, so its vector instructions count.  Measured at
// 16384 x 256 on one MI355X: 20.0 -> 19.75 us (the one-item form measured
// slower with it and keeps the division).
template <class Est, int L, int OPT>
__global__ void __launch_bounds__(256) duo_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr int K = 4;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  constexpr int G = 64 / L;   // rows per item
  constexpr int SPAN = L * K;  // row length
  static_assert(!Tr::kDual, "one recurrence per pass");
  static_assert(G * SPAN == kDuoItem, "an item is whole rows");

  // B's first NL streams go through LDS (at most three: 12 KiB per block, so
  // eight blocks fit a CU's LDS with room to spare); the rest -> registers
  constexpr int NL = NS < 3 ? NS : 3;
  __shared__ float s_b[4][NL][kDuoItem];  // each wave's second item, memory order

  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int team = lane / L;  // row of the item
  const int g = lane & (L - 1);
  const bool team_first_lane = g == 0;
  const uint32_t cs = REV ? (uint32_t)(SPAN - (g + 1) * K) : (uint32_t)(g * K);  // column of the lane's chunk
  const uint32_t lds_idx = (uint32_t)(team * SPAN) + cs;
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
  for (int st = 0; st < NS; ++st) load_s<F32S, K, true>(srcs[st], ra * T, cs, 0u, da.s[st]);
  if constexpr (USE_FLAGS) {
    load_flag_raw<K, true>(p.term + ra * T, cs, 0u, fta);
    load_flag_raw<K, true>(p.trunc + ra * T, cs, 0u, fra);
  }
  da.rowv = load1<F32S>(p.row, ra, 0u);

  // ---- 2. item B: streams -> LDS (lane l moves elements 4 l .. 4 l + 3 of the
  // item, clamped into the array), flags and row value -> registers
  {
    int64_t e = item_bc * kDuoItem + 4 * lane;
    if (e > E * T - 4) e = E * T - 4;
#pragma unroll
    for (int st = 0; st < NL; ++st)
      __builtin_amdgcn_global_load_lds((gbl_void_ptr)(srcs[st] + e), (lds_void_ptr)&s_b[w][st][0], 16, 0, 0);
  }
  LaneIn<Est, K> db;
#pragma unroll
  for (int st = NL; st < NS; ++st) load_s<F32S, K, true>(srcs[st], rb * T, cs, 0u, db.s[st]);
  unsigned ftb[K], frb[K];
  if constexpr (USE_FLAGS) {
    load_flag_raw<K, true>(p.term + rb * T, cs, 0u, ftb);
    load_flag_raw<K, true>(p.trunc + rb * T, cs, 0u, frb);
  }
  db.rowv = load1<F32S>(p.row, rb, 0u);

  // ---- 3. A's flags and bootstrap gather
  unsigned tba = 0, rba = 0, tbb = 0, rbb = 0;
#pragma unroll
  for (int m = 0; m < K; ++m) da.tb[m] = db.tb[m] = 0.0f;
  if constexpr (USE_FLAGS) {
    tba = flag_bits<K, true>(fta) & tmask;
    rba = flag_bits<K, true>(fra) & rmask;
  }
  if constexpr (GATHER_TB) {
    if ((rba & ~tba) != 0u && p.has_tboot) load_chunk<K, true>(p.tboot + ra * T, cs, 0u, da.tb);
  }

  // ---- 4. everything landed (B's DMA included); B's flags and gather
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  if constexpr (USE_FLAGS) {
    tbb = flag_bits<K, true>(ftb) & tmask;
    rbb = flag_bits<K, true>(frb) & rmask;
  }
  if constexpr (GATHER_TB) {
    if ((rbb & ~tbb) != 0u && p.has_tboot) load_chunk<K, true>(p.tboot + rb * T, cs, 0u, db.tb);
  }

  // ---- 5. item A
  {
    double C = 0.0;
    if constexpr (!Tr::kBackwardRl) C = (ok_a && p.has_row) ? (double)da.rowv : 0.0;
    PredIn carry{0.0f, 0.0, 0u};  // a row is one tile: no scan predecessor
    float o0[K], o1[K];
    stream_tile<Est, L, K, false, Tr::kRetrace>(da, sc, tba, rba, cs, T, team_first_lane, lane, C, carry, o0, o1);
    if (G == 1 || ok_a) {
      store_s<F32S, K, true>(p.out0, ra * T, cs, K, o0);
      if constexpr (OUT1) store_s<F32S, K, true>(p.out1, ra * T, cs, K, o1);
    }
  }

  // ---- 6. item B
  if (!has_b) return;
#pragma unroll
  for (int st = 0; st < NL; ++st) lds_read4<F32S>(&s_b[w][st][lds_idx], db.s[st]);
  {
    double C = 0.0;
    if constexpr (!Tr::kBackwardRl) C = (ok_b && p.has_row) ? (double)db.rowv : 0.0;
    PredIn carry{0.0f, 0.0, 0u};
    float o0[K], o1[K];
    stream_tile<Est, L, K, false, Tr::kRetrace>(db, sc, tbb, rbb, cs, T, team_first_lane, lane, C, carry, o0, o1);
    if (G == 1 || ok_b) {
      store_s<F32S, K, true>(p.out0, rb * T, cs, K, o0);
      if constexpr (OUT1) store_s<F32S, K, true>(p.out1, rb * T, cs, K, o1);
    }
  }
}

}  // namespace rlscan
