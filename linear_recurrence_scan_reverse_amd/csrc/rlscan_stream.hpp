// rlscan_stream.hpp -- the streaming kernel: a loader wave feeds compute waves
// through an LDS ring (gfx950 global->LDS DMA), for rows made of whole,
// aligned tiles.
//
// Why: the scan is HBM-bound, and keeping enough bytes in flight (~64 KiB per
// CU at ~5.5 TB/s) decides the speed.  A wave that both loads and stores
// cannot keep loads in flight across its stores (gfx9 has one memory counter,
// so waiting for any load also drains pending stores and every later load),
// and data in flight held in VGPRs costs occupancy.  So each wave gets one
// kind of memory traffic:
//   * the loader (wave 0) only issues global->LDS DMA (global_load_lds): the
//     flag bytes of an item one tick before its input streams and row
//     values; its waits are exact counts and the data occupies no VGPRs;
//   * the gather wave (wave 1, estimators with truncation bootstraps) reads
//     the landed flags from LDS, copies them next to the item's data and
//     DMAs the bootstrap of every truncated step (lanes without one fetch a
//     single shared, cache-resident line), so that gather never stalls a
//     compute wave;
//   * the compute waves read LDS, scan and store; they never wait on memory.
// Time advances in ticks separated by s_barrier.  At tick t compute wave c
// scans item t of its own item sequence from data slot t % S, while the
// loader fills items t + P (data) and t + P + 1 (flags) and the gather wave
// serves item t + 2.
//
// An item is 64*K consecutive elements of every [E,T] array: G = 64 / L whole
// rows when a row is a single tile (T == L * K), or one tile of one row.  A
// compute wave walks the tiles of a row in scan order and carries the running
// value and the boundary inputs (V_{t+1} / EQ_{t+1}, c_{t+1}, done_{t-1})
// across tiles in registers.
#pragma once

#include "rlscan_kernel.hpp"

namespace rlscan {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;

// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 0x3) << 14));
}
// s_waitcnt lgkmcnt(0) only.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14)); }

// Block barrier without the memory fences of __syncthreads (which would drain
// the loader's in-flight DMA); the empty asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void tick_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class Est, int K, bool FLAGS>
struct StreamCfg {
  using Tr = Traits<Est>;
  static constexpr int NS = Tr::kStreams;
  static constexpr bool USE_FLAGS = FLAGS && Tr::kUsesFlags;
  static constexpr bool GATHER = USE_FLAGS && Tr::kBackwardRl;  // a gather wave, early flags
  static constexpr int N = 64 * K;          // elements per item
  static constexpr int P = NS >= 5 ? 2 : 3;  // items the data DMA runs ahead
  static constexpr int S = P + 1;           // data ring slots
  static constexpr int SF = 4;              // early-flag ring slots: flags of item j land from tick j-4 to j-2
  // bytes of one data slot (streams, bootstraps, flags, row values) and of the flag ring
  static constexpr int kSlotBytes = 4 * NS * N + (GATHER ? 4 * N : 0) + (USE_FLAGS ? 2 * N : 0) + 16;
  static constexpr int kFlagBytes = GATHER ? 2 * N : 0;
  static constexpr int kPerWave = S * kSlotBytes + SF * kFlagBytes;
  // compute waves per block: fill half of the 160 KiB LDS (two blocks per CU)
  static constexpr int kLdsBudget = 80 * 1024;
  // DMA instructions per item and compute wave: data (+ flags when not early), early flags, gather
  static constexpr int kOpsData = NS * (K / 4) + 1 + ((USE_FLAGS && !GATHER) ? 2 * (K / 4) : 0);
  static constexpr int kOpsFlags = GATHER ? 2 * (K / 4) : 0;
  static constexpr int kOpsGather = GATHER ? K / 4 : 0;
  // Loader schedule (see the kernel): DMA ops per compute wave that stay in
  // flight at each of its waits.  With early flags: before the start-up
  // barrier (flags 0..3 and data 0 issued, flags 0-1 complete), before the
  // first tick (data 0 complete), and every tick (data t+1 and flags t+3
  // complete while flags t+4 and data t+P were issued last).
  static constexpr int kWaitPre1 = 2 * kOpsFlags + kOpsData;
  static constexpr int kWaitPre0 = (P - 1) * kOpsData;
  static constexpr int kWaitTick = GATHER ? (P == 3 ? 2 * kOpsData + kOpsFlags : kOpsFlags + kOpsData)
                                          : (P - 1) * kOpsData;
  static constexpr int kWaitMax = kWaitPre1 > kWaitPre0 ? (kWaitPre1 > kWaitTick ? kWaitPre1 : kWaitTick)
                                                        : (kWaitPre0 > kWaitTick ? kWaitPre0 : kWaitTick);
  static constexpr int NC_LDS = kLdsBudget / kPerWave;
  static constexpr int NC_VM = 63 / kWaitMax;
  static constexpr int NC_RAW = NC_LDS < NC_VM ? NC_LDS : NC_VM;
  static constexpr int NC = NC_RAW > 7 ? 7 : (NC_RAW < 1 ? 1 : NC_RAW);
  static constexpr int kHelpers = GATHER ? 2 : 1;  // loader (+ gather wave)
  static constexpr int kThreads = 64 * (NC + kHelpers);
};

template <class Est, int K, bool FLAGS>
struct Slot {
  using C = StreamCfg<Est, K, FLAGS>;
  float s[C::NS][C::N];
  float tb[C::GATHER ? C::N : 1];
  unsigned fl[C::USE_FLAGS ? 2 : 1][C::USE_FLAGS ? C::N / 4 : 1];  // raw flag bytes, 4 per word
  float rowv[4];
};

template <class Est, int K, bool FLAGS>
struct FlagSlot {
  using C = StreamCfg<Est, K, FLAGS>;
  unsigned fl[2][C::GATHER ? C::N / 4 : 1];
};

// Template parameters: estimator tag, team width L (16, 32 or 64 lanes per
// row), chunk K (4 or 8 steps per lane), OPT (bit 0: flags present; bit 1:
// second output).  Requires T % (L * K) == 0, L < 64 only when T == L * K,
// every dense array aligned to 16 bytes, and T < 2^26.
template <class Est, int L, int K, int OPT>
__global__ void __launch_bounds__((StreamCfg<Est, K, (OPT & 1) != 0>::kThreads))
stream_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  using Cfg = StreamCfg<Est, K, (OPT & 1) != 0>;
  using SlotT = Slot<Est, K, (OPT & 1) != 0>;
  using FlagT = FlagSlot<Est, K, (OPT & 1) != 0>;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Cfg::NS;
  constexpr int NC = Cfg::NC;
  constexpr int S = Cfg::S;
  constexpr int SF = Cfg::SF;
  constexpr int P = Cfg::P;
  constexpr int G = 64 / L;    // rows per item when a row is one tile
  constexpr int SPAN = L * K;  // tile length
  constexpr bool USE_FLAGS = Cfg::USE_FLAGS;
  constexpr bool GATHER = Cfg::GATHER;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr int FIRST_COMPUTE = Cfg::kHelpers;
  static_assert(K % 4 == 0 && K <= 8, "chunk of 4 or 8 steps");
  static_assert(P == 2 || P == 3, "lead of two or three items");
  static_assert(S * NC * sizeof(SlotT) + SF * NC * sizeof(FlagT) <= 96 * 1024, "LDS ring");

  __shared__ SlotT ring[S][NC];
  __shared__ FlagT fring[SF][NC];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t T = p.T;
  const int64_t E = p.E;
  const uint32_t T32 = (uint32_t)T;
  const int64_t ntiles = T / SPAN;      // (the host guarantees T % SPAN == 0)
  const int64_t nrg = (E + G - 1) / G;  // row groups (items of one tile)
  const int64_t ncw = (int64_t)gridDim.x * NC;
  const int64_t cw0 = (int64_t)blockIdx.x * NC;  // first compute wave of this block
  // block-uniform tick count: the block's first compute wave has the most row groups
  const int64_t ticks = (cw0 < nrg ? (nrg - cw0 + ncw - 1) / ncw : 0) * ntiles;

  // An item position (the same for every compute wave of the block): the j-th
  // row group of the wave, ts-th tile in scan order, with the ring slots it
  // uses.  Advanced by one per tick (no divisions: their temporaries would
  // force waits on in-flight memory operations).
  struct Cursor {
    int64_t j, ts;
    int slot, fslot;
  };
  auto advance = [&](Cursor q) __attribute__((always_inline)) {
    if (++q.ts == ntiles) {
      q.ts = 0;
      ++q.j;
    }
    q.slot = q.slot + 1 == S ? 0 : q.slot + 1;
    q.fslot = q.fslot + 1 == SF ? 0 : q.fslot + 1;
    return q;
  };
  auto item_rg = [&](int c, const Cursor& q) { return cw0 + c + q.j * ncw; };
  auto item_tile = [&](const Cursor& q) { return REV ? ntiles - 1 - q.ts : q.ts; };
  const int64_t last_rg = nrg - 1;
  // element index of an item's first element, rows past E clamped
  auto item_base = [&](int c, const Cursor& cur, int64_t& base) {
    int64_t rg = item_rg(c, cur);
    rg = rg < last_rg ? rg : last_rg;
    base = (G > 1) ? rg * G * T : rg * T + item_tile(cur) * SPAN;
    return rg;
  };
  // element offset of this lane's q-th 4-element group inside the item (G > 1
  // only when T == SPAN, so rows split at the constant SPAN); rows past E read
  // row E - 1
  auto lane_off = [&](int64_t rg, int q) -> uint32_t {
    const uint32_t f = (uint32_t)(q * 256 + lane * 4);
    if constexpr (G > 1) {
      const int64_t row = rg * G + f / SPAN;
      if (row >= E) return (uint32_t)((E - 1 - rg * G) * SPAN + f % SPAN);
    }
    return f;
  };

  if (wave == 0) {
    // ================================================================ loader
    // Tick t issues the flags of item t+4 (early-flag estimators) and the data
    // of item t+P; before the barrier that ends tick t, the data of item t+1
    // and the flags of item t+3 are complete.
    const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};
    auto issue_flags = [&](const Cursor& cur) __attribute__((always_inline)) {
      if constexpr (GATHER) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          int64_t base;
          const int64_t rg = item_base(c, cur, base);
          FlagT& fs = fring[cur.fslot][c];
#pragma unroll
          for (int q = 0; q < K / 4; ++q) {
            const uint32_t off = lane_off(rg, q);
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.term + base + off), (lds_void_ptr)&fs.fl[0][q * 64], 4,
                                             0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.trunc + base + off), (lds_void_ptr)&fs.fl[1][q * 64], 4,
                                             0, 0);
          }
        }
      }
    };
    auto issue_data = [&](const Cursor& cur) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        int64_t base;
        const int64_t rg = item_base(c, cur, base);
        SlotT& sl = ring[cur.slot][c];
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const uint32_t off = lane_off(rg, q);
#pragma unroll
          for (int st = 0; st < NS; ++st)
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)at(srcs[st] + base, off), (lds_void_ptr)&sl.s[st][q * 256],
                                             16, 0, 0);
          if constexpr (USE_FLAGS && !GATHER) {
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.term + base + off), (lds_void_ptr)&sl.fl[0][q * 64], 4,
                                             0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.trunc + base + off), (lds_void_ptr)&sl.fl[1][q * 64], 4,
                                             0, 0);
          }
        }
        // row values: lane i (< G) lands in rowv[i]; the DMA writes one word per active
        // lane, so the other lanes stay off
        if (lane < G) {
          int64_t row = rg * G + lane;
          row = row < E ? row : E - 1;
          __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.row + row), (lds_void_ptr)&sl.rowv[0], 4, 0, 0);
        }
      }
    };
    Cursor cd{0, 0, 0, 0};
    if constexpr (GATHER) {
      Cursor cf = cd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // flags of items 0..3
        issue_flags(cf);
        cf = advance(cf);
      }
      issue_data(cd);  // data of item 0
      cd = advance(cd);
      wait_vmcnt<NC * Cfg::kWaitPre1>();  // flags of items 0, 1 complete
      tick_barrier();                     // start-up barrier: the gather wave serves items 0, 1
#pragma unroll
      for (int i = 1; i < P; ++i) {
        issue_data(cd);
        cd = advance(cd);
      }
      wait_vmcnt<NC * Cfg::kWaitPre0>();  // data of item 0 (and flags of item 2) complete
      tick_barrier();
      for (int64_t t = 0; t < ticks; ++t) {
        issue_flags(cf);
        cf = advance(cf);
        issue_data(cd);
        cd = advance(cd);
        wait_vmcnt<NC * Cfg::kWaitTick>();
        tick_barrier();
      }
    } else {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        issue_data(cd);
        cd = advance(cd);
      }
      wait_vmcnt<NC * Cfg::kWaitPre0>();  // data of item 0 complete
      tick_barrier();
      for (int64_t t = 0; t < ticks; ++t) {
        issue_data(cd);
        cd = advance(cd);
        wait_vmcnt<NC * Cfg::kWaitTick>();
        tick_barrier();
      }
    }
    wait_vmcnt<0>();  // no DMA into this block's LDS may outlive the block
  } else if (GATHER && wave == 1) {
    // ================================================================ gather wave
    // Tick t serves item t+2 (its flags landed before the barrier that opened
    // tick t); before the barrier that ends tick t, item t+1 is complete.
    auto serve = [&](const Cursor& cur) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        int64_t base;
        const int64_t rg = item_base(c, cur, base);
        SlotT& sl = ring[cur.slot][c];
        const FlagT& fs = fring[cur.fslot][c];
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const unsigned w_t = fs.fl[0][q * 64 + lane];
          const unsigned w_r = fs.fl[1][q * 64 + lane];
          sl.fl[0][q * 64 + lane] = w_t;
          sl.fl[1][q * 64 + lane] = w_r;
          // some step truncated and not terminated (nonzero byte of w_r over a zero byte of w_t)
          const unsigned m_t = w_t & (p.has_term ? ~0u : 0u);
          const unsigned m_r = w_r & (p.has_trunc ? ~0u : 0u);
          const unsigned nz_t = (((m_t & 0x7f7f7f7fu) + 0x7f7f7f7fu) | m_t) & 0x80808080u;
          const unsigned nz_r = (((m_r & 0x7f7f7f7fu) + 0x7f7f7f7fu) | m_r) & 0x80808080u;
          const bool need = (nz_r & ~nz_t) != 0u && p.has_tboot;
          const float* src = need ? at(p.tboot + base, lane_off(rg, q)) : p.tboot;
          __builtin_amdgcn_global_load_lds((gbl_void_ptr)src, (lds_void_ptr)&sl.tb[q * 256], 16, 0, 0);
        }
      }
    };
    Cursor cg{0, 0, 0, 0};
    tick_barrier();  // start-up barrier: flags of items 0, 1 have landed
    serve(cg);
    cg = advance(cg);
    serve(cg);
    cg = advance(cg);
    wait_vmcnt<NC * Cfg::kOpsGather>();  // item 0 complete
    wait_lgkm0();
    tick_barrier();
    for (int64_t t = 0; t < ticks; ++t) {
      serve(cg);
      cg = advance(cg);
      wait_vmcnt<NC * Cfg::kOpsGather>();
      wait_lgkm0();
      tick_barrier();
    }
    wait_vmcnt<0>();
  } else {
    // ================================================================ compute
    const int c = wave - FIRST_COMPUTE;
    const int team = lane / L;  // row of the item (G > 1); 0 when L == 64
    const int g = lane & (L - 1);
    const bool team_first_lane = (g == 0);
    const uint32_t cs_local = REV ? (uint32_t)(SPAN - (g + 1) * K) : (uint32_t)(g * K);
    const uint32_t lds_idx = (uint32_t)(team * SPAN) + cs_local;  // element index inside the item
    const double gamma = p.gamma, lam = p.lam, gl = gamma * lam;
    const ScanScalars sc{gamma, lam, gl, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0, p.has_tboot != 0};
    const unsigned tmask = p.has_term ? ~0u : 0u;
    const unsigned rmask = p.has_trunc ? ~0u : 0u;
    constexpr int MLAST = REV ? 0 : K - 1;

    double C = 0.0;
    PredIn carry{0.0f, 0.0, 0u};  // boundary inputs handed from the previous tile of the row

    tick_barrier();
    if constexpr (GATHER) tick_barrier();  // the gather wave's start-up tick
    Cursor cur{0, 0, 0, 0};
    for (int64_t t = 0; t < ticks; ++t, cur = advance(cur)) {
      const SlotT& sl = ring[cur.slot][c];
      const int64_t rg = item_rg(c, cur);
      const int64_t tile = item_tile(cur);
      const bool first_tile = cur.ts == 0;
      const int64_t row = rg * G + team;
      const bool row_ok = row < E;
      const uint32_t cs = (uint32_t)(tile * SPAN) + cs_local;

      LaneIn<Est, K> d;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&sl.s[st][lds_idx + 4 * q]);
          d.s[st][4 * q + 0] = v.x; d.s[st][4 * q + 1] = v.y; d.s[st][4 * q + 2] = v.z; d.s[st][4 * q + 3] = v.w;
        }
      }
      if constexpr (GATHER) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&sl.tb[lds_idx + 4 * q]);
          d.tb[4 * q + 0] = v.x; d.tb[4 * q + 1] = v.y; d.tb[4 * q + 2] = v.z; d.tb[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int m = 0; m < K; ++m) d.tb[m] = 0.0f;
      }
      d.rowv = sl.rowv[team];
      unsigned tbits = 0, rbits = 0;
      if constexpr (USE_FLAGS) {
        unsigned tw[K / 4], rw[K / 4];
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          tw[q] = sl.fl[0][lds_idx / 4 + q];
          rw[q] = sl.fl[1][lds_idx / 4 + q];
        }
        tbits = flag_bits_words<K / 4>(tw) & tmask;
        rbits = flag_bits_words<K / 4>(rw) & rmask;
      }

      if (first_tile) {
        if constexpr (Tr::kBackwardRl) C = 0.0;
        else C = (row_ok && p.has_row) ? (double)d.rowv : 0.0;
        carry = PredIn{0.0f, 0.0, 0u};
      }
      const LanePairs<K> lp = build_pairs<Est, K, true>(d, sc, tbits, rbits, cs, T, K, team_first_lane, carry);
      const AB incl = lane_scan<L>(fold_lane<K>(lp.e));
      const double y_last = __builtin_fma(incl.a, C, incl.b);
      const double from_below = shift_up_f64(y_last);
      const double x_in = team_first_lane ? C : from_below;
      const double C_next = group_last_f64<L>(y_last, lane);
      double xs[K];
      rewalk<K>(lp.e, x_in, xs);
      float o0[K], o1[K];
      epilogue<Est, K>(d, lp, sc, x_in, xs, o0, o1);

      // boundary inputs for the next tile of this row (held by the scan-last lane, 63)
      if constexpr (L == 64) {
        if constexpr (Tr::kRetrace) {
          const double ratio = (double)d.s[3][MLAST] / (double)d.s[4][MLAST];
          const double cl = lam * (ratio < 1.0 ? ratio : 1.0);
          carry.v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, d.s[2][MLAST]), 63));
          const unsigned long long u = __builtin_bit_cast(unsigned long long, cl);
          const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, 63);
          const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), 63);
          carry.c = __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
        } else if constexpr (Tr::kNbValue) {
          carry.v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, d.s[1][MLAST]), 63));
        } else if constexpr (Tr::kNbDone) {
          carry.done = (unsigned)__builtin_amdgcn_readlane((int)(((tbits | rbits) >> MLAST) & 1u), 63);
        }
      }
      C = C_next;

      if (row_ok) {
        const int64_t eb = rg * G * T;  // element index of the item's first row
        const uint32_t off = (uint32_t)team * T32 + cs;
        store_chunk<K, true>(p.out0 + eb, off, K, o0);
        if constexpr (OUT1) store_chunk<K, true>(p.out1 + eb, off, K, o1);
      }
      wait_lgkm0();
      tick_barrier();
    }
  }
}

}  // namespace rlscan
