// rlscan_stream.hpp -- the streaming kernel: a loader wave feeds compute waves
// through LDS rings (gfx950 global->LDS DMA), for rows made of whole,
// aligned tiles of 4 L steps.
//
// Why: the scan is HBM-bound, and keeping enough bytes in flight (~64 KiB per
// CU at ~5.5 TB/s) decides the speed.  A wave that both loads and stores
// cannot keep loads in flight across its stores (gfx9 has one memory counter,
// so waiting for any load also drains pending stores and every later load),
// and data in flight held in VGPRs costs occupancy.  So each wave gets one
// kind of memory traffic:
//   * the loader (wave 0) only issues global->LDS DMA: flag bytes, input
//     streams and row values.  Its waits are exact counts of its own DMA
//     instructions (they complete in issue order), and the data occupies no
//     VGPRs;
//   * the gather wave (wave 1, estimators with truncation bootstraps) reads
//     landed flags from LDS and DMAs the bootstrap of every truncated step
//     (lanes without one issue an out-of-range buffer DMA that touches no
//     memory);
//   * the compute waves read LDS, scan and store; they never wait on memory.
//
// Time advances in ticks separated by s_barrier; at tick t every compute wave
// scans item t of its own item sequence.  Under load the memory system is a
// queue about P ticks deep (whatever is issued lands about P ticks later), so
// every stage gets a lead of P ticks:
//   data of item t+P               issued by the loader at tick t,
//   bootstrap gather of item t+P   issued by the gather wave at tick t, from the
//   flags of item t+2P             issued by the loader at tick t.
// Before tick 0 the loader issues the flags of items 0..2P-1 and the data of
// items 0..P-1 in one burst, and the gather wave serves items 0..P-1 in P
// warm-up ticks as their flags land.
//
// An item is 256 consecutive elements of every [E,T] array: G = 64 / L whole
// rows when a row is a single tile (T == 4 L), or one tile of one row.  A
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

// vmcnt <= n for a wave-uniform run-time n (s_waitcnt takes only an
// immediate, so this is a jump table); n is clamped to [0, 63].
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n <= 0 ? 0 : (n >= 63 ? 63 : n)) {
#define RLSCAN_WAIT_CASE(i) \
  case i:                   \
    wait_vmcnt<i>();        \
    break;
#define RLSCAN_WAIT_CASE8(i)                                                                     \
  RLSCAN_WAIT_CASE(i) RLSCAN_WAIT_CASE(i + 1) RLSCAN_WAIT_CASE(i + 2) RLSCAN_WAIT_CASE(i + 3) \
  RLSCAN_WAIT_CASE(i + 4) RLSCAN_WAIT_CASE(i + 5) RLSCAN_WAIT_CASE(i + 6) RLSCAN_WAIT_CASE(i + 7)
    RLSCAN_WAIT_CASE8(0)
    RLSCAN_WAIT_CASE8(8)
    RLSCAN_WAIT_CASE8(16)
    RLSCAN_WAIT_CASE8(24)
    RLSCAN_WAIT_CASE8(32)
    RLSCAN_WAIT_CASE8(40)
    RLSCAN_WAIT_CASE8(48)
    RLSCAN_WAIT_CASE8(56)
#undef RLSCAN_WAIT_CASE8
#undef RLSCAN_WAIT_CASE
    default:
      break;
  }
}

// Block barrier without the memory fences of __syncthreads (which would drain
// the loader's in-flight DMA); the empty asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void tick_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kStreamItem = 256;  // elements per item (64 lanes x 4 steps)

// Size of the gather wave's buffer resources, and the offset that lies past
// them: any in-row offset of an item and the next one is smaller (rows hold
// fewer than 2^30 elements of at most 4 bytes).
constexpr uint32_t kOutOfRangeOffset = 0xFFFFFFF0u;

// Most compute waves per block for an estimator.  Measured at 16384 x 256
// (two blocks per CU, lead 2): a power of two that splits the rows evenly over
// the blocks beats filling the LDS for the light estimators, while V-trace and
// Retrace are fastest with as many waves as the LDS holds.  The estimators
// with a gather wave run best with 4 (discounted returns: 14.5 us with 8
// compute waves, 11.5 us with 4).
template <class Est>
constexpr int stream_nc_cap() {
  if constexpr (__is_same(Est, Vtrace) || __is_same(Est, Retrace)) return 16;
  if constexpr (__is_same(Est, TdLambda) || __is_same(Est, Gae) || __is_same(Est, ReturnsTdLambda) ||
                __is_same(Est, DiscountedReturn))
    return 4;
  return 8;
}

template <class Est, bool FLAGS, int P_, int BPC, class Fmt = F32S>
struct StreamCfg {
  using Tr = Traits<Est>;
  using ET = typename Fmt::T;                 // stored element type
  static constexpr int ES = (int)sizeof(ET);  // bytes per stored value
  static constexpr int IPD = 4 / ES;          // items per 16-byte-per-lane DMA (16-bit: two)
  static constexpr int NS = Tr::kStreams;
  static constexpr bool USE_FLAGS = FLAGS && Tr::kUsesFlags;
  static constexpr bool GATHER = USE_FLAGS && Tr::kBackwardRl;  // a gather wave
  static constexpr int N = kStreamItem;
  static constexpr int P = P_;                       // data lead (ticks)
  static constexpr int LG = GATHER ? P : 0;          // gather lead
  static constexpr int LF = LG + P;                  // flag lead
  static constexpr int S = P + 1;                    // data ring slots
  static constexpr int SF = USE_FLAGS ? LF + 1 : 1;  // flag ring slots
  static constexpr int kHelpers = GATHER ? 2 : 1;    // loader (+ gather wave)
  static constexpr int kLdsBudget = 160 * 1024 / BPC;
  // LDS bytes for nc compute waves (16 bytes of slack per slot for padding)
  static constexpr int lds_bytes(int nc) {
    const int slot = ES * NS * nc * N + (GATHER ? ES * nc * N : 0) + 16 * nc + 16;
    const int fslot = USE_FLAGS ? 2 * nc * N : 16;
    return S * slot + SF * fslot;
  }
  // DMA instructions per tick of the loader: flags (16 B per lane, four items
  // per instruction and array), data (one per stream and IPD items) and row
  // values; and of the gather wave (one per IPD items)
  static constexpr int fops(int nc) { return USE_FLAGS ? 2 * ((nc + 3) / 4) : 0; }
  static constexpr int dops(int nc) { return NS * ((nc + IPD - 1) / IPD) + 1; }
  static constexpr int gops(int nc) { return (nc + IPD - 1) / IPD; }
  // most DMA instructions the loader ever has in flight: after the start-up
  // burst, and right after a steady-state issue
  static constexpr int max_inflight(int nc) {
    const int a = LF * fops(nc) + P * dops(nc);
    const int b = P * (fops(nc) + dops(nc));
    return a > b ? a : b;
  }
  static constexpr int pick_nc() {
    int best = 1;
    for (int nc = 1; nc + kHelpers <= 16 && nc <= stream_nc_cap<Est>(); ++nc)
      if (lds_bytes(nc) <= kLdsBudget && max_inflight(nc) <= 63 && (!GATHER || P * gops(nc) <= 63)) best = nc;
    return best;
  }
  static constexpr int NC = pick_nc();
  static constexpr int F = fops(NC);
  static constexpr int D = dops(NC);
  static constexpr int kThreads = 64 * (NC + kHelpers);
  static_assert(max_inflight(NC) <= 63, "loader DMA in flight must fit the 6-bit counter");
};

// One tick's data for all compute waves of a block (values in the stored
// format; a row value is the 4-byte word holding it).
template <class Cfg>
struct alignas(16) TickSlot {
  typename Cfg::ET s[Cfg::NS][Cfg::NC][Cfg::N];
  typename Cfg::ET tb[Cfg::GATHER ? Cfg::NC : 1][Cfg::GATHER ? Cfg::N : 1];
  uint32_t rowv[Cfg::NC * 4];
};

// K = 4 stored values at an LDS element address, widened.
template <class Fmt>
__device__ __forceinline__ void lds_read4(const typename Fmt::T* q, float (&o)[4]) {
  if constexpr (__is_same(Fmt, F32S)) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(q);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    const unsigned long long v = *reinterpret_cast<const unsigned long long*>(q);
    const uint32_t w0 = (uint32_t)v, w1 = (uint32_t)(v >> 32);
    o[0] = s_to_f32<Fmt>((uint16_t)w0); o[1] = s_to_f32<Fmt>((uint16_t)(w0 >> 16));
    o[2] = s_to_f32<Fmt>((uint16_t)w1); o[3] = s_to_f32<Fmt>((uint16_t)(w1 >> 16));
  }
}

// Address of element bidx + off of a value array of ES-byte elements.
template <int ES>
__device__ __forceinline__ const void* elem_addr(const float* base, int64_t bidx, uint32_t off) {
  return reinterpret_cast<const char*>(base) + ES * bidx + (uint32_t)(off * (uint32_t)ES);
}
// One tick's flag bytes (terminated, truncated) for all compute waves.
template <class Cfg>
struct alignas(16) FlagTick {
  uint8_t fl[Cfg::USE_FLAGS ? 2 : 1][Cfg::USE_FLAGS ? Cfg::NC : 1][Cfg::USE_FLAGS ? Cfg::N : 4];
};

// One lane's part of one tile of one row: pairs, wave scan, re-walk and
// outputs.  C is the row's running value (in: beyond this tile; out: beyond
// the next one), `carry` the boundary inputs handed between tiles of the row.
// FASTDIV as for build_pairs.  CARRY: the next tile of the same rows follows (rows longer than one tile):
// the boundary inputs it needs are taken from the scan-last lane of each team
// (lane 63 with one team per wave; with several teams per wave only when
// CARRY_TEAMS is set, where rows of L < 64 lanes span several tiles).
template <class E2, int L, int K, bool CARRY = true, bool FASTDIV = false, bool CARRY_TEAMS = false>
__device__ __forceinline__ void stream_tile(const LaneIn<E2, K>& d, const ScanScalars& sc, unsigned tbits,
                                            unsigned rbits, uint32_t cs, int64_t T, bool team_first_lane, int lane,
                                            double& C, PredIn& carry, float (&o0)[K], float (&o1)[K]) {
  using Tr = Traits<E2>;
  constexpr int MLAST = E2::kReverse ? 0 : K - 1;
  const LanePairs<K> lp = build_pairs<E2, K, true, FASTDIV>(d, sc, tbits, rbits, cs, T, K, team_first_lane, carry);
  const AB incl = lane_scan<L>(fold_lane<K>(lp.e));
  const double y_last = __builtin_fma(incl.a, C, incl.b);
  const double from_below = shift_up_f64(y_last);
  const double x_in = team_first_lane ? C : from_below;
  const double C_next = group_last_f64<L>(y_last, lane);
  double xs[K];
  rewalk<K>(lp.e, x_in, xs);
  epilogue<E2, K>(d, lp, sc, x_in, xs, o0, o1);

  // boundary inputs for the next tile of this row (held by the scan-last lane, 63)
  if constexpr (CARRY && L == 64) {
    if constexpr (Tr::kRetrace) {
      const double ratio = (double)d.s[3][MLAST] / (double)d.s[4][MLAST];
      const double cl = sc.lam * (ratio < 1.0 ? ratio : 1.0);
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
  } else if constexpr (CARRY && CARRY_TEAMS) {
    // several teams per wave: each team's scan-last lane (team start + L - 1)
    const int src = (lane & ~(L - 1)) + L - 1;
    if constexpr (Tr::kRetrace) {
      const double ratio = (double)d.s[3][MLAST] / (double)d.s[4][MLAST];
      carry.v = __shfl(d.s[2][MLAST], src, 64);
      carry.c = __shfl(sc.lam * (ratio < 1.0 ? ratio : 1.0), src, 64);
    } else if constexpr (Tr::kNbValue) {
      carry.v = __shfl(d.s[1][MLAST], src, 64);
    } else if constexpr (Tr::kNbDone) {
      carry.done = (unsigned)__shfl((int)(((tbits | rbits) >> MLAST) & 1u), src, 64);
    }
  }
  C = C_next;
}

// Template parameters: estimator tag, team width L (16, 32 or 64 lanes per
// row), OPT (bit 0: flags present; bit 1: second output), data lead P, blocks
// per CU the LDS is split for, storage format.  Requires T % (4 L) == 0,
// L < 64 only when T == 4 L, every dense array and flag array aligned to 16
// bytes, and T < 2^30 (checked by the C ABI); 16-bit formats also need the
// row-value array 4-byte aligned and E even (row values travel as the 4-byte
// word holding them).
template <class Est, int L, int OPT, int P, int BPC, class Fmt = F32S>
__global__ void __launch_bounds__((StreamCfg<Est, (OPT & 1) != 0, P, BPC, Fmt>::kThreads))
stream_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  using Cfg = StreamCfg<Est, (OPT & 1) != 0, P, BPC, Fmt>;
  using SlotT = TickSlot<Cfg>;
  using FlagT = FlagTick<Cfg>;
  constexpr int K = 4;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Cfg::NS;
  constexpr int NC = Cfg::NC;
  constexpr int S = Cfg::S;
  constexpr int SF = Cfg::SF;
  constexpr int LG = Cfg::LG;
  constexpr int LF = Cfg::LF;
  constexpr int G = 64 / L;    // rows per item when a row is one tile
  constexpr int SPAN = L * K;  // tile length
  constexpr bool USE_FLAGS = Cfg::USE_FLAGS;
  constexpr bool GATHER = Cfg::GATHER;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr int FIRST_COMPUTE = Cfg::kHelpers;
  constexpr int ES = Cfg::ES;    // bytes per stored value
  constexpr int IPD = Cfg::IPD;  // items per 16-byte-per-lane DMA
  static_assert(!Tr::kDual || ES == 4, "the two-output pass stores float32");
  static_assert(P >= 1 && P <= 4, "lead of one to four items");
  static_assert(NC * G <= 64, "one row-value DMA per tick");
  static_assert(S * sizeof(SlotT) + SF * sizeof(FlagT) <= (size_t)Cfg::kLdsBudget, "LDS rings");

  __shared__ SlotT ring[S];
  __shared__ FlagT fring[SF];

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
  const int ticks = (int)((cw0 < nrg ? (nrg - cw0 + ncw - 1) / ncw : 0) * ntiles);

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
  auto item_tile = [&](const Cursor& q) { return REV ? ntiles - 1 - q.ts : q.ts; };
  const int64_t last_rg = nrg - 1;
  // element index of the first element of compute wave c's item, rows past E clamped
  auto item_base = [&](int64_t c, const Cursor& cur, int64_t& base) {
    int64_t rg = cw0 + c + cur.j * ncw;
    rg = rg < last_rg ? rg : last_rg;
    base = (G > 1) ? rg * G * T : rg * T + item_tile(cur) * SPAN;
    return rg;
  };
  // offset of element f of an item (G > 1 only when T == SPAN, so rows split
  // at the constant SPAN); rows past E read row E - 1
  auto elem_off = [&](int64_t rg, uint32_t f) -> uint32_t {
    if constexpr (G > 1) {
      const int64_t row = rg * G + f / SPAN;
      if (row >= E) return (uint32_t)((E - 1 - rg * G) * SPAN + f % SPAN);
    }
    return f;
  };

  if (wave == 0) {
    // ================================================================ loader
    constexpr int F = Cfg::F, D = Cfg::D;
    const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};
    // flags of one tick: instruction q, lane l -> item 4q + l/16, bytes 16 (l%16) ..
    auto issue_flags = [&](const Cursor& cur) __attribute__((always_inline)) {
      if constexpr (USE_FLAGS) {
#pragma unroll
        for (int q = 0; q < (NC + 3) / 4; ++q) {
          const int c = 4 * q + (lane >> 4);
          if (c < NC) {
            int64_t base;
            const int64_t rg = item_base(c, cur, base);
            const uint32_t off = elem_off(rg, (uint32_t)(lane & 15) * 16);
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.term + base + off),
                                             (lds_void_ptr)&fring[cur.fslot].fl[0][4 * q][0], 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)(p.trunc + base + off),
                                             (lds_void_ptr)&fring[cur.fslot].fl[1][4 * q][0], 16, 0, 0);
          }
        }
      }
    };
    // data: one DMA per stream moves 16 bytes per lane, i.e. one float32 item
    // (64 lanes x 4 values) or two 16-bit items (lanes 32..63 take the next
    // compute wave's item, which follows in LDS)
    auto issue_data = [&](const Cursor& cur) __attribute__((always_inline)) {
      SlotT& sl = ring[cur.slot];
      const int ci_off = IPD == 2 ? (lane >> 5) : 0;
      const uint32_t li = IPD == 2 ? (uint32_t)(lane & 31) : (uint32_t)lane;
#pragma unroll
      for (int c = 0; c < NC; c += IPD) {
        const int ci = c + ci_off;
        if (ci < NC) {  // (an odd NC leaves the upper half of the last 16-bit DMA idle)
          int64_t base;
          const int64_t rg = item_base(ci, cur, base);
          const uint32_t off = elem_off(rg, li * (16 / ES));
#pragma unroll
          for (int st = 0; st < NS; ++st)
            __builtin_amdgcn_global_load_lds((gbl_void_ptr)elem_addr<ES>(srcs[st], base, off),
                                             (lds_void_ptr)&sl.s[st][c][0], 16, 0, 0);
        }
      }
      // row values: lane c*G + g -> row g of compute wave c's item (16-bit: the
      // aligned word holding it)
      if (lane < NC * G) {
        int64_t base;
        const int64_t rg = item_base(lane / G, cur, base);
        int64_t row = rg * G + lane % G;
        row = row < E ? row : E - 1;
        const void* src = ES == 4 ? (const void*)(p.row + row)
                                  : (const void*)(reinterpret_cast<const uint32_t*>(p.row) + (row >> 1));
        __builtin_amdgcn_global_load_lds((gbl_void_ptr)src, (lds_void_ptr)&sl.rowv[0], 4, 0, 0);
      }
    };
    // start-up burst: flags of items 0..LF-1, then data of items 0..P-1
    const int LFv = ticks < LF ? ticks : LF;
    const int Pv = ticks < P ? ticks : P;
    Cursor cf{0, 0, 0, 0}, cd{0, 0, 0, 0};
    for (int k = 0; k < LFv; ++k) {
      issue_flags(cf);
      cf = advance(cf);
    }
    for (int k = 0; k < Pv; ++k) {
      issue_data(cd);
      cd = advance(cd);
    }
    int cum = LFv * F + Pv * D;  // DMA instructions issued so far
    // warm-up ticks: before the barrier that ends warm-up tick w (w = -LG-1 .. -1)
    // the flags of item w+LG+1 have landed, and at w = -1 also the data of item 0
#pragma unroll
    for (int w = -LG - 1; w <= -1; ++w) {
      const int k = w + LG + 1;
      int n = cum;
      if (USE_FLAGS && k < LFv) n = cum - (k + 1) * F;
      if (w == -1) n = (Pv - 1) * D < n ? (Pv - 1) * D : n;
      wait_vmcnt_dyn(n);
      tick_barrier();
    }
    // steady ticks: issue flags of item t+LF and data of item t+P; before the
    // barrier that ends tick t the data of item t+1 has landed, and with it
    // (issued no later) the flags of item t+1+LG
    int hist[P];  // hist[i]: DMA instructions issued up to the end of tick t-i
#pragma unroll
    for (int i = 0; i < P; ++i) hist[i] = 0;
    for (int t = 0; t < ticks; ++t) {
      if (t + LF < ticks) {
        issue_flags(cf);
        cf = advance(cf);
        cum += F;
      }
      if (t + P < ticks) {
        issue_data(cd);
        cd = advance(cd);
        cum += D;
      }
#pragma unroll
      for (int i = P - 1; i > 0; --i) hist[i] = hist[i - 1];
      hist[0] = cum;
      if (t + 1 < ticks) {
        const int req = (t + 1 < P) ? LFv * F + (t + 2) * D : hist[P - 1];
        wait_vmcnt_dyn(cum - req);
      }
      tick_barrier();
    }
    wait_vmcnt<0>();  // no DMA into this block's LDS may outlive the block
  } else if (GATHER && wave == 1) {
    // ================================================================ gather wave
    // Serves item k at tick k-LG (warm-up ticks for k < LG): reads its landed
    // flags and DMAs the bootstrap chunk of every lane that has a truncated,
    // not terminated step.  Before the barrier that ends tick t, the gather
    // of item t+1 has landed.
    constexpr int GO = Cfg::gops(NC);  // DMA instructions per served item-tick
    auto serve = [&](const Cursor& cur) __attribute__((always_inline)) {
      SlotT& sl = ring[cur.slot];
      const FlagT& fs = fring[cur.fslot];
      // the same lane -> item mapping as the data DMA: a lane covers 16 / ES steps
      const int ci_off = IPD == 2 ? (lane >> 5) : 0;
      const uint32_t li = IPD == 2 ? (uint32_t)(lane & 31) : (uint32_t)lane;
#pragma unroll
      for (int c = 0; c < NC; c += IPD) {
        const int ci = c + ci_off;
        if (ci < NC) {
          int64_t base;
          const int64_t rg = item_base(ci, cur, base);
          // some step truncated and not terminated (a nonzero truncated byte over
          // a zero terminated byte), over the lane's flag words
          unsigned nz = 0;
#pragma unroll
          for (int h = 0; h < 4 / ES; ++h) {
            const unsigned w_t = reinterpret_cast<const unsigned*>(&fs.fl[0][ci][0])[li * (4 / ES) + h];
            const unsigned w_r = reinterpret_cast<const unsigned*>(&fs.fl[1][ci][0])[li * (4 / ES) + h];
            const unsigned m_t = w_t & (p.has_term ? ~0u : 0u);
            const unsigned m_r = w_r & (p.has_trunc ? ~0u : 0u);
            const unsigned nz_t = (((m_t & 0x7f7f7f7fu) + 0x7f7f7f7fu) | m_t) & 0x80808080u;
            const unsigned nz_r = (((m_r & 0x7f7f7f7fu) + 0x7f7f7f7fu) | m_r) & 0x80808080u;
            nz |= nz_r & ~nz_t;
          }
          const bool need = nz != 0u && p.has_tboot;
          // A buffer resource based at item c's first element (lanes of item
          // c + 1 in a 16-bit instruction lie one item further): lanes without
          // a bootstrap to fetch pass an offset past its range and touch no
          // memory.  (Re-reading their rewards instead, an L2 hit, measured
          // 0.5-0.8 us slower for discounted returns at 16384 x 256.)
          int64_t base0;
          (void)item_base(c, cur, base0);
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<char*>(reinterpret_cast<const char*>(p.tboot)) + ES * base0, 0, (int)kOutOfRangeOffset,
              0x00020000);
          const uint32_t off = (uint32_t)(ES * (base - base0 + elem_off(rg, li * (16 / ES))));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)&sl.tb[c][0], 16, need ? off : kOutOfRangeOffset,
                                                   0, 0, 0);
        }
      }
    };
    // gathers allowed in flight at the end of tick w: those of items w+2 .. min(w+LG, ticks-1)
    auto after = [&](int w) {
      const int hi = (w + LG < ticks - 1) ? w + LG : ticks - 1;
      const int n = hi - (w + 1);
      return n > 0 ? n * GO : 0;
    };
    Cursor cg{0, 0, 0, 0};
#pragma unroll
    for (int w = -LG - 1; w <= -1; ++w) {
      if (w >= -LG && w + LG < ticks) {
        serve(cg);
        cg = advance(cg);
      }
      if (w == -1) wait_vmcnt_dyn(after(w));
      tick_barrier();
    }
    for (int t = 0; t < ticks; ++t) {
      if (t + LG < ticks) {
        serve(cg);
        cg = advance(cg);
      }
      if (t + 1 < ticks) wait_vmcnt_dyn(after(t));
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
    double C = 0.0;
    PredIn carry{0.0f, 0.0, 0u};  // boundary inputs handed from the previous tile of the row
    double C2 = 0.0;               // the second recurrence of a two-output pass
    PredIn carry2{0.0f, 0.0, 0u};

#pragma unroll
    for (int w = -LG - 1; w <= -1; ++w) tick_barrier();
    Cursor cur{0, 0, 0, 0};
    for (int t = 0; t < ticks; ++t, cur = advance(cur)) {
      const SlotT& sl = ring[cur.slot];
      const int64_t rg = cw0 + c + cur.j * ncw;
      const int64_t tile = item_tile(cur);
      const bool first_tile = cur.ts == 0;
      const int64_t row = rg * G + team;
      const bool row_ok = row < E;
      const uint32_t cs = (uint32_t)(tile * SPAN) + cs_local;

      LaneIn<Est, K> d;
#pragma unroll
      for (int st = 0; st < NS; ++st) lds_read4<Fmt>(&sl.s[st][c][lds_idx], d.s[st]);
      if constexpr (GATHER) {
        lds_read4<Fmt>(&sl.tb[c][lds_idx], d.tb);
      } else {
#pragma unroll
        for (int m = 0; m < K; ++m) d.tb[m] = 0.0f;
      }
      {
        const uint32_t wv = sl.rowv[c * G + team];
        if constexpr (ES == 4) {
          d.rowv = __builtin_bit_cast(float, wv);
        } else {
          const int64_t rw = row_ok ? row : E - 1;  // the row the loader fetched
          d.rowv = s_to_f32<Fmt>((uint16_t)((rw & 1) ? (wv >> 16) : wv));
        }
      }
      unsigned tbits = 0, rbits = 0;
      if constexpr (USE_FLAGS) {
        const FlagT& fs = fring[cur.fslot];
        const unsigned tw[1] = {*reinterpret_cast<const unsigned*>(&fs.fl[0][c][lds_idx])};
        const unsigned rw[1] = {*reinterpret_cast<const unsigned*>(&fs.fl[1][c][lds_idx])};
        tbits = flag_bits_words<1>(tw) & tmask;
        rbits = flag_bits_words<1>(rw) & rmask;
      }

      if (first_tile) {
        if constexpr (Tr::kBackwardRl) C = 0.0;
        else C = (row_ok && p.has_row) ? (double)d.rowv : 0.0;
        carry = PredIn{0.0f, 0.0, 0u};
        C2 = 0.0;
        carry2 = PredIn{0.0f, 0.0, 0u};
      }
      float o0[K], o1[K];
      if constexpr (Tr::kDual) {
        // discounted return (rewards only) and TD(lambda) return (rewards, values)
        LaneIn<DiscountedReturn, K> da;
        LaneIn<TdLambda, K> db;
#pragma unroll
        for (int m = 0; m < K; ++m) {
          da.s[0][m] = d.s[0][m];
          db.s[0][m] = d.s[0][m];
          db.s[1][m] = d.s[1][m];
          da.tb[m] = db.tb[m] = d.tb[m];
        }
        da.rowv = db.rowv = d.rowv;
        float unused[K];
        stream_tile<DiscountedReturn, L, K>(da, sc, tbits, rbits, cs, T, team_first_lane, lane, C, carry, o0, unused);
        stream_tile<TdLambda, L, K>(db, sc, tbits, rbits, cs, T, team_first_lane, lane, C2, carry2, o1, unused);
      } else {
        stream_tile<Est, L, K>(d, sc, tbits, rbits, cs, T, team_first_lane, lane, C, carry, o0, o1);
      }

      if (row_ok) {
        const int64_t eb = rg * G * T;  // element index of the item's first row
        const uint32_t off = (uint32_t)team * T32 + cs;
        store_s<Fmt, K, true>(p.out0, eb, off, K, o0);
        if constexpr (OUT1) store_s<Fmt, K, true>(p.out1, eb, off, K, o1);
      }
      wait_lgkm0();
      tick_barrier();
    }
  }
}

}  // namespace rlscan
