// rlscan_tmitem.hpp -- time-major [T, E] arrays scanned in the row-major item
// layout: loader waves move chunks of 64 steps x 64 (or 32) environments
// between HBM and LDS, and compute waves read a chunk back as rows (4
// environments x 64 steps per item, 16 lanes x 4 steps per row), run the
// per-lane code of the row-major kernels on them, carrying each row across
// chunks, and leave the outputs in LDS for the loaders to store.
//
// The time-major kernel in rlscan_timemajor.hpp maps lanes to environments
// and splits time over the 16 waves of a block, so a block computes only once
// all its waves' loads have landed, and at 16384 environments (one block per
// CU) loads and compute never overlap.  Here a block owns 64 or 32
// environments and walks their time chunk by chunk, one chunk per tick, with
// the loads of the next three chunks in flight while one is scanned.  Every
// environment's whole time range stays with one compute wave, so no wave
// waits for another's result; the waves of a block meet once per tick, at a
// barrier.
//
// Tick s (chunks in scan order; backward estimators walk time from the end):
//   loaders  store the outputs of chunk s-1 (read back from LDS), write chunk
//            s+1's streams and chunk s+2's flags (requested two ticks earlier)
//            to LDS and request chunk s+3's streams and s+4's flags into the
//            registers those left;
//   compute  read chunk s+1's flags and request its truncation bootstraps,
//            scan chunk s (its flags and bootstraps taken a tick earlier) and
//            write its outputs over its streams in LDS.
// Each wave only touches its own LDS cells of a slot (the loaders by step, the
// compute waves by environment), and a slot changes hands only at a barrier.
// Global accesses take whole runs of a step: 16 bytes a lane for streams and
// outputs (scattered 16-byte stores of the compute waves' rows cost three
// times the kernel's time), 4 bytes for flags, through buffer resources over
// one chunk; requests of chunks before the first or past the last get a
// resource of no records and touch no memory, so no branch surrounds a
// request.  LDS holds every array environment-major (the loaders transpose on
// the way in and out): a lane reads its 4 steps of a stream with two 8-byte
// reads, and its 4 steps of both flags as one word (the loaders fold the two
// flag bytes of a step into one, bit 0 terminated, bit 1 truncated).
// Against step-major LDS rows read a step at a time, at 16384 x 256:
// discounted returns 14.1 -> 12.5 us.
#pragma once

#include "rlscan_duo.hpp"
#include "rlscan_stream.hpp"

namespace rlscan {

constexpr int kTiChunk = 64;   // steps per chunk (a row tile: 16 lanes x 4 steps)
constexpr int kTiSlots = 2;    // chunks of streams in LDS (3 or 4, loads further ahead, measured slower)
constexpr int kTiRow = 66;     // LDS words per environment and stream of a chunk (64 steps, padded)
// A block of EB environments (64 or 32): EB / 8 compute waves of two items
// (4 environments each), EB / 16 loader waves, each 64 / (EB / 16) steps of
// every chunk; 16-byte lane accesses cover a step's EB environments with
// EB / 4 lanes.
template <int EB>
constexpr int ti_compute() { return EB / 8; }
template <int EB>
constexpr int ti_loaders() { return EB / 16; }
template <int EB>
constexpr int ti_threads() { return 64 * (ti_compute<EB>() + ti_loaders<EB>()); }
// LDS words per environment of a chunk's flags (16 words of 4 steps, padded
// so the loaders' writes spread over the banks)
template <int EB>
constexpr int ti_flag_row() { return EB == 64 ? 17 : 18; }

// Wait until this wave's LDS accesses are done (lgkmcnt 0; the vector-memory
// and export counters are left alone), so a barrier after it publishes them.
__device__ __forceinline__ void lds_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Bit 0 of every byte of x: whether the byte is non-zero.
__device__ __forceinline__ uint32_t bytes_nonzero(uint32_t x) {
  return ((((x & 0x7f7f7f7fu) + 0x7f7f7f7fu) | x) >> 7) & 0x01010101u;
}

// Template parameters: estimator (one recurrence, at most three input
// streams, or Retrace's five with 32 environments per block: the LDS holds
// two chunks of them), OPT as for the other kernels, EB environments per
// block, S the storage format (16-bit values are widened to float32 on the
// way into LDS and rounded back, to nearest even, on the way out).  E a
// positive multiple of EB, T a positive multiple of 64, every per-step array
// 16-byte aligned, 64 * E * 4 < 2^31 (checked by the launcher).  Block b: environments
// EB b .. EB b + EB - 1.
template <class Est, int OPT, int EB, class S = F32S>
__global__ void __launch_bounds__(ti_threads<EB>()) tm_item_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr int L = 16, K = 4, SPAN = kTiChunk;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr int NOUT = OUT1 ? 2 : 1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  static_assert(!Tr::kDual && NOUT <= NS, "one recurrence, outputs over streams");
  static_assert(NS <= 3 || (NS == 5 && EB == 32), "five streams (Retrace) in blocks of 32 environments");
  static_assert(EB == 64 || EB == 32, "blocks of 64 or 32 environments");
  constexpr int NSL = kTiSlots, NFL = NSL + 1;
  constexpr int NC = ti_compute<EB>(), NLD = ti_loaders<EB>(), FROW = ti_flag_row<EB>();
  constexpr int ES = __is_same(S, F32S) ? 4 : 2;  // bytes per stored value
  constexpr int LB = 4 * ES;       // bytes per lane access of values (4 environments)
  constexpr int LPR = EB / 4;      // lanes per step of a value access
  // chunks of loads in flight in a loader's registers; against one (chunk
  // s+2 requested in tick s, written in tick s+1), two gave float32 4096 x 512
  // TD(lambda) 14.3 -> 13.2 us, 16384 x 512 discounted returns 19.7 -> 18.5,
  // bfloat16 4096 x 256 V-trace 12.4 -> 11.5 (bfloat16 V-trace from 16384
  // environments 2-4% slower); three or four needed more registers than the
  // block allows and spilled
  constexpr int PD = 2;
  constexpr int SPI = 64 / LPR;    // steps per loader instruction

  // streams (then outputs) of NSL chunks: [slot][stream][environment][step]
  __shared__ __attribute__((aligned(16))) float s_d[NSL][NS][EB][kTiRow];
  // flags of NSL + 1 chunks, one byte per step (bit 0 terminated, bit 1
  // truncated), four steps a word: [slot][environment][steps / 4]
  __shared__ uint32_t s_f[USE_FLAGS ? NFL : 1][USE_FLAGS ? EB : 1][FROW];
  // slots of chunk s (s >= -1)
  auto dslot = [](int s) { return (s + NSL) % NSL; };
  auto fslot = [](int s) { return s % NFL; };

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t E = p.E, T = p.T;
  const int ticks = (int)(T / SPAN);
  const int64_t e0 = xcd_group(blockIdx.x, gridDim.x, 128 / EB) * EB;
  // resource over chunk s of an [T, E] array of esz-byte elements, from the
  // block's first environment; no records for s outside [0, ticks)
  auto chunk_rs = [&](const void* base, int s, int esz) {
    const bool on = s >= 0 && s < ticks;
    const int64_t t0 = on ? (REV ? (int64_t)(ticks - 1 - s) : (int64_t)s) * SPAN : 0;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(base)) + (t0 * E + e0) * esz, 0, on ? (int)(SPAN * E * esz) : 0,
        0x00020000);
  };

  if (wave >= NC) {
    // ================================================================ loaders
    const int lw = wave - NC;
    const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};
    float* dsts[2] = {p.out0, p.out1};
    // streams and outputs: access q of a lane covers step SPI (lw + NLD q) +
    // lane / LPR, environments 4 (lane % LPR) .. + 3
    const int scol = 4 * (lane % LPR);
    auto dstep = [&](int q) { return SPI * (lw + NLD * q) + lane / LPR; };
    auto doff = [&](int q) { return (uint32_t)(((int64_t)dstep(q) * E + scol) * ES); };
    // flags: steps 4 fword .. + 3, environments 4 (lane % LPR) .. + 3, one
    // 4-byte access per step and array
    const int fword = (16 / NLD) * lw + lane / LPR;
    auto foff = [&](int m) { return (uint32_t)((int64_t)(4 * fword + m) * E + scol); };

    typedef typename RawOf<LB>::T Chunk[NS][4];
    typedef uint32_t Flags[2][4];
    auto issue_data = [&](int s, Chunk& x) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const __amdgpu_buffer_rsrc_t rs = chunk_rs(srcs[st], s, ES);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[st][q] = raw_buffer_load<LB>(rs, doff(q));
      }
    };
    auto write_data = [&](int s, const Chunk& x) {
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float f[4];
          if constexpr (LB == 16) unpack16<S, 4>(x[st][q], f);
          else unpack8<S, 4>(x[st][q], f);
          const int t = dstep(q);
#pragma unroll
          for (int j = 0; j < 4; ++j) s_d[dslot(s)][st][scol + j][t] = f[j];
        }
    };
    auto issue_flags = [&](int s, Flags& f) {
      if constexpr (USE_FLAGS) {
        const __amdgpu_buffer_rsrc_t rt = chunk_rs(p.term, s, 1), rr = chunk_rs(p.trunc, s, 1);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f[0][m] = __builtin_amdgcn_raw_buffer_load_b32(rt, foff(m), 0, 2);
          f[1][m] = __builtin_amdgcn_raw_buffer_load_b32(rr, foff(m), 0, 2);
        }
      }
    };
    // the lane's 4 steps x 4 environments of flags, combined and turned to
    // one word of 4 steps per environment
    auto write_flags = [&](int s, const Flags& f) {
      if constexpr (USE_FLAGS) {
        uint32_t c[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) c[m] = bytes_nonzero(f[0][m]) | (bytes_nonzero(f[1][m]) << 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = ((c[0] >> (8 * j)) & 0xffu) | (((c[1] >> (8 * j)) & 0xffu) << 8) |
                             (((c[2] >> (8 * j)) & 0xffu) << 16) | (((c[3] >> (8 * j)) & 0xffu) << 24);
          s_f[fslot(s)][scol + j][fword] = w;
        }
      }
    };
    // outputs of chunk s (left over its streams by the compute waves)
    auto store_out = [&](int s) {
#pragma unroll
      for (int o = 0; o < NOUT; ++o) {
        const __amdgpu_buffer_rsrc_t rs = chunk_rs(dsts[o], s, ES);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = dstep(q);
          float f[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) f[j] = s_d[dslot(s)][o][scol + j][t];
          if constexpr (LB == 16) raw_buffer_store<16>(__builtin_bit_cast(u32x4, (f32x4){f[0], f[1], f[2], f[3]}), rs, doff(q));
          else raw_buffer_store<8>(pack8<S, 4>(f), rs, doff(q));
        }
      }
    };
    auto loaded = [] {
      lds_done();
      tick_barrier();
    };
    // Register sets in flight: chunk k's streams and flags sit in set k % PD
    // from their request until written to LDS.  Tick s writes chunk s+1's
    // streams (into the slot chunk s-1's outputs just left) and chunk s+2's
    // flags, and requests chunk s+1+PD's and s+2+PD's into the sets those
    // free, so PD chunks of loads are in flight behind the one being scanned.
    auto tick = [&](int s, Chunk& X, Flags& F) {
      store_out(s - 1);
      write_data(s + 1, X);
      issue_data(s + 1 + PD, X);
      write_flags(s + 2, F);
      issue_flags(s + 2 + PD, F);
      loaded();
    };

    Chunk x[PD];
    Flags f[PD];
    // before the first tick: the streams and flags of chunks 0 .. PD-1
    // requested at once; chunk 0's streams and chunks 0 and 1's flags in LDS
    // (their sets refilled with chunks PD and PD+1)
#pragma unroll
    for (int k = 0; k < PD; ++k) issue_flags(k, f[k]);
#pragma unroll
    for (int k = 0; k < PD; ++k) issue_data(k, x[k]);
    asm volatile("" ::: "memory");
    write_flags(0, f[0]);
    issue_flags(PD, f[0]);
    write_flags(1, f[1]);
    issue_flags(PD + 1, f[1]);
    write_data(0, x[0]);
    issue_data(PD, x[0]);
    loaded();
    // whole rounds of PD ticks (static set indices), then the rest
    int base = 0;
    for (; base + PD <= ticks; base += PD) {
#pragma unroll
      for (int k = 0; k < PD; ++k) tick(base + k, x[(k + 1) % PD], f[(k + 2) % PD]);
    }
#pragma unroll
    for (int k = 0; k + 1 < PD; ++k)
      if (base + k < ticks) tick(base + k, x[(k + 1) % PD], f[(k + 2) % PD]);
    store_out(ticks - 1);
  } else {
    // ================================================================ compute
    const int c = wave;
    const int team = lane / L;  // row (environment) of the item
    const int g = lane & (L - 1);
    const bool team_first_lane = g == 0;
    const uint32_t cs_local = REV ? (uint32_t)(SPAN - (g + 1) * K) : (uint32_t)(g * K);
    const double gamma = p.gamma, lam = p.lam;
    const ScanScalars sc{gamma, lam, gamma * lam, (float)p.rho_bar, (float)p.c_bar, p.has_row != 0,
                         p.has_tboot != 0};
    const unsigned tmask = p.has_term ? ~0u : 0u;
    const unsigned rmask = p.has_trunc ? ~0u : 0u;
    // 16-bit formats: the fast Retrace quotient and V-trace exp, as in the
    // other kernels of those formats
    constexpr bool FAST = Tr::kRetrace || !__is_same(S, F32S);

    int col[2];     // environment offset inside the block, per item
    float rowv[2];  // bootstrap value / init of the environment
    double C[2];
    PredIn carry[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      col[it] = 8 * c + 4 * it + team;
      rowv[it] = p.has_row ? load1<S>(p.row, e0, (uint32_t)col[it]) : 0.0f;
      C[it] = 0.0;
      if constexpr (!Tr::kBackwardRl) C[it] = p.has_row ? (double)rowv[it] : 0.0;
      carry[it] = PredIn{0.0f, 0.0, 0u};
    }

    // what a chunk's scan takes besides its streams: the lane's flag bits and
    // truncation bootstraps, per item (read a tick ahead)
    struct Side {
      unsigned tb[2], rb[2];
      float boot[2][K];
    };
    // flags of chunk s from LDS, and its bootstraps requested (none past the
    // last chunk; lanes and steps without one pass an offset outside the resource)
    auto side_of = [&](int s, Side& o) {
      const int sf = s < ticks ? s : ticks - 1;  // flags slot read (any valid one past the end)
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        o.tb[it] = o.rb[it] = 0u;
        if constexpr (USE_FLAGS) {
          const uint32_t w = s_f[fslot(sf)][col[it]][cs_local / 4];
          o.tb[it] = ((w & 1u) | ((w >> 7) & 2u) | ((w >> 14) & 4u) | ((w >> 21) & 8u)) & tmask;
          o.rb[it] = (((w >> 1) & 1u) | ((w >> 8) & 2u) | ((w >> 15) & 4u) | ((w >> 22) & 8u)) & rmask;
        }
#pragma unroll
        for (int m = 0; m < K; ++m) o.boot[it][m] = 0.0f;
      }
      if constexpr (GATHER_TB) {
        const __amdgpu_buffer_rsrc_t rs = chunk_rs(p.tboot, s, ES);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const unsigned need = p.has_tboot ? (o.rb[it] & ~o.tb[it]) : 0u;
#pragma unroll
          for (int m = 0; m < K; ++m) {
            const uint32_t off = (uint32_t)(((int64_t)(cs_local + m) * E + col[it]) * ES);
            const uint32_t at = ((need >> m) & 1u) ? off : kDuoOff;
            if constexpr (ES == 4)
              o.boot[it][m] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, at, 0, 2));
            else
              o.boot[it][m] = s_to_f32<S>(__builtin_amdgcn_raw_buffer_load_b16(rs, at, 0, 2));
          }
        }
      }
    };
    // one tick: chunk s+1's side inputs requested, chunk s scanned, its
    // outputs written over its streams
    auto tick = [&](int s, const Side& cur, Side& nxt) {
      side_of(s + 1, nxt);
      const int slot = dslot(s);
      const int64_t t0 = (REV ? (int64_t)(ticks - 1 - s) : (int64_t)s) * SPAN;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        LaneIn<Est, K> d;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const f32x2* q = reinterpret_cast<const f32x2*>(&s_d[slot][st][col[it]][cs_local]);
          const f32x2 a = q[0], b = q[1];
          d.s[st][0] = a.x;
          d.s[st][1] = a.y;
          d.s[st][2] = b.x;
          d.s[st][3] = b.y;
        }
#pragma unroll
        for (int m = 0; m < K; ++m) d.tb[m] = cur.boot[it][m];
        d.rowv = rowv[it];
        float o0[K], o1[K];
        stream_tile<Est, L, K, true, FAST, true>(d, sc, cur.tb[it], cur.rb[it], (uint32_t)t0 + cs_local, T,
                                                 team_first_lane, lane, C[it], carry[it], o0, o1);
        f32x2* w0 = reinterpret_cast<f32x2*>(&s_d[slot][0][col[it]][cs_local]);
        w0[0] = (f32x2){o0[0], o0[1]};
        w0[1] = (f32x2){o0[2], o0[3]};
        if constexpr (OUT1) {
          f32x2* w1 = reinterpret_cast<f32x2*>(&s_d[slot][1][col[it]][cs_local]);
          w1[0] = (f32x2){o1[0], o1[1]};
          w1[1] = (f32x2){o1[2], o1[3]};
        }
      }
      lds_done();
      tick_barrier();
    };

    Side sa, sb;
    tick_barrier();  // chunk 0 and the flags of chunks 0 and 1 are in LDS
    side_of(0, sa);
    // Tick 0 runs ahead of the loop, so the loop is entered from the same
    // point of the pipeline its back edge returns to (the compiler's count of
    // requests in flight then agrees on both, and its waits stay exact); the
    // two side-input register sets swap roles from tick to tick.
    tick(0, sa, sb);
    for (int s = 1; s < ticks; s += 2) {
      tick(s, sb, sa);
      if (s + 1 < ticks) tick(s + 1, sa, sb);
    }
  }
}

}  // namespace rlscan
