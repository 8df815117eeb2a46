// rlscan_tmdma.hpp -- the item form of the time-major path with its loads
// moved by the global->LDS DMA of gfx950: a chunk of 64 steps x EB
// environments lands in LDS step-major, exactly as it lies in HBM (1 KiB
// groups, one per DMA request of a wave), so no register holds it in flight
// and no wave transposes it.  Compute waves read a lane's 4 steps of an
// environment from 4 step rows of a group, scan them as the register item
// form does (same per-lane code, same carries) and write the outputs back over
// the first streams; storer waves read the outputs back 16 bytes a lane (whole
// runs of a step) and store them.
//
// Waves of a block of EB environments: EB / 8 compute waves (two items of 4
// environments each), EB / 32 DMA waves and EB / 32 storer waves.  The DMA and
// storer roles are separate waves because the compiler makes any LDS read of a
// wave wait for all of that wave's DMA requests still in flight.
//
// Chunk c (scan order) sits in data slot c % NSL: requested by the DMA waves
// in tick c - NSL + 2, scanned in tick c, stored in tick c + 1, so NSL - 2
// chunks are in flight behind the one scanned.  Its flags (the raw bytes of
// both arrays) sit in flag slot c % (NSL - 1): requested in tick c - NSL + 1,
// with chunk c - 1's streams, and read by the compute waves in tick c - 1 (a
// tick ahead, to request the truncation bootstraps; chunk 0's before the
// prologue's second barrier).  Every DMA wave waits, before each tick's
// barrier, until what the next tick reads has landed: its requests of NSL - 3
// later ticks may stay in flight.
#pragma once

#include "rlscan_tmitem.hpp"

namespace rlscan {

constexpr int kTdGroup = 1040;  // LDS bytes per 1 KiB DMA group (16 bytes of padding rotate the banks)

template <int EB> constexpr int td_compute() { return EB / 8; }
template <int EB> constexpr int td_dma() { return EB / 32; }
template <int EB> constexpr int td_storers() { return EB / 32; }
template <int EB> constexpr int td_threads() { return 64 * (td_compute<EB>() + td_dma<EB>() + td_storers<EB>()); }
// 1 KiB groups per stream chunk (64 steps of EB values of es bytes) and per flag array chunk
constexpr int td_groups(int eb, int es) { return eb * es * 64 / 1024; }
constexpr int td_flag_groups(int eb) { return eb * 64 / 1024; }
// rf: flags through the storer waves' registers, combined one byte a step
// (three slots of the register item form's words) instead of DMA
constexpr int td_lds_bytes(int ns, int eb, int es, int nsl, bool flags, bool rf = false) {
  return nsl * ns * td_groups(eb, es) * kTdGroup +
         (!flags ? 0 : rf ? 3 * eb * (eb == 64 ? 17 : 18) * 4 : (nsl - 1) * 2 * td_flag_groups(eb) * kTdGroup);
}
// DMA requests of one DMA wave per tick
constexpr int td_requests(int ns, int eb, int es, bool flags, bool rf = false) {
  return (ns * td_groups(eb, es) + (flags && !rf ? 2 * td_flag_groups(eb) : 0)) / (eb / 32);
}
constexpr int kTdLdsBudget = 160 * 1024;
// Whether NSL data slots fit: the LDS, and a DMA wave's wait count (6 bits).
constexpr bool td_fits(int ns, int eb, int es, int nsl, bool flags, bool rf = false) {
  return nsl >= 3 && td_lds_bytes(ns, eb, es, nsl, flags, rf) <= kTdLdsBudget &&
         (nsl - 2) * td_requests(ns, eb, es, flags, rf) < 64;
}

// Template parameters as for tm_item_kernel, plus NSL data slots (3 or more)
// and RF: the flags moved by the storer waves through registers (4-byte
// accesses, two chunks ahead, both bytes of a step folded into one, as the
// register item form does) instead of by DMA, for three streams whose raw
// flag bytes do not fit beside three data slots.
// E a positive multiple of EB, T a positive multiple of 64, every per-step
// array 16-byte aligned, 64 * E * 4 < 2^31 (checked by the launcher).
template <class Est, int OPT, int EB, class S, int NSL, bool RF = false>
__global__ void __launch_bounds__(td_threads<EB>()) tm_dma_kernel(const KernelArgs p) {
  using Tr = Traits<Est>;
  constexpr int L = 16, K = 4, SPAN = kTiChunk;
  constexpr bool REV = Est::kReverse;
  constexpr int NS = Tr::kStreams;
  constexpr bool USE_FLAGS = (OPT & 1) && Tr::kUsesFlags;
  constexpr bool OUT1 = (OPT & 2) && Tr::kHasOut1;
  constexpr int NOUT = OUT1 ? 2 : 1;
  constexpr bool GATHER_TB = USE_FLAGS && Tr::kBackwardRl;
  constexpr bool DMAF = USE_FLAGS && !RF, RFL = USE_FLAGS && RF;  // flags by DMA / through registers
  static_assert(!Tr::kDual && NOUT <= NS, "one recurrence, outputs over streams");
  static_assert(EB == 64 || EB == 32, "blocks of 64 or 32 environments");
  constexpr int ES = (int)sizeof(typename S::T);
  constexpr int RB = EB * ES;     // bytes of one step's EB values
  constexpr int SPI = 1024 / RB;  // steps per group of a stream
  constexpr int NQ = 64 / SPI;    // groups per stream chunk
  constexpr int LPR = RB / 16;    // lanes per step of a 16-byte access
  constexpr int SPF = 1024 / EB;  // steps per group of a flag array
  constexpr int NQF = 64 / SPF;   // groups per flag array chunk
  constexpr int LPF = EB / 16;    // lanes per step of a flag access
  constexpr int NFL = NSL - 1;
  constexpr int NC = td_compute<EB>(), ND = td_dma<EB>(), NST = td_storers<EB>();
  static_assert(td_fits(NS, EB, ES, NSL, USE_FLAGS, RF), "slots fit the LDS and the wait count");
  static_assert(NQ % ND == 0 && NQ % NST == 0 && (2 * NQF) % ND == 0, "groups split evenly over waves");
  constexpr int WAITN = (NSL - 3) * td_requests(NS, EB, ES, USE_FLAGS, RF);
  constexpr int WAIT0 = (NSL - 2) * td_requests(NS, EB, ES, USE_FLAGS, RF);  // after chunk 0's flags
  constexpr int FROW = ti_flag_row<EB>();

  // streams (then outputs) of NSL chunks: [slot][stream][group][bytes], a
  // group holding SPI steps of EB values each
  __shared__ __attribute__((aligned(16))) unsigned char s_d[NSL][NS][NQ][kTdGroup];
  // flag bytes of NFL chunks: [slot][array: terminated, truncated][group][bytes]
  __shared__ __attribute__((aligned(16))) unsigned char s_f[DMAF ? NFL : 1][2][DMAF ? NQF : 1][kTdGroup];
  // (RF) flags of three chunks, one byte a step (bit 0 terminated, bit 1
  // truncated), four steps a word: [slot][environment][steps / 4]
  __shared__ uint32_t s_fw[RFL ? 3 : 1][RFL ? EB : 1][FROW];

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
  // a lane's 16-byte access of group q of a stream chunk: step q SPI + lane / LPR,
  // environments (lane % LPR) 16 / ES .. + 16 / ES - 1
  auto data_off = [&](int q) {
    return (uint32_t)(((int64_t)(q * SPI + lane / LPR) * E + (lane % LPR) * (16 / ES)) * ES);
  };

  if (wave >= NC + ND) {
    // ================================================================ storers
    const int sw = wave - NC - ND;
    float* dsts[2] = {p.out0, p.out1};
    auto store_out = [&](int s) {
      const int slot = (s + NSL) % NSL;
#pragma unroll
      for (int o = 0; o < NOUT; ++o) {
        const __amdgpu_buffer_rsrc_t rs = chunk_rs(dsts[o], s, ES);
#pragma unroll
        for (int i = 0; i < NQ / NST; ++i) {
          const int q = sw + NST * i;
          const u32x4 v = *reinterpret_cast<const u32x4*>(&s_d[slot][o][q][lane * 16]);
          raw_buffer_store<16>(v, rs, data_off(q));
        }
      }
    };
    // (RF) flags: two passes of 4-byte accesses, each covering steps 4 fword ..
    // + 3 of environments scol .. scol + 3; chunk k's words in register set k % 2
    constexpr int FLPR = EB / 4;  // lanes per step row of a 4-byte flag access
    const int scol = 4 * (lane % FLPR);
    auto fword = [&](int i) { return (16 / NST) * sw + (64 / FLPR) * i + lane / FLPR; };
    typedef uint32_t Flags[2][2][4];
    auto issue_flags = [&](int c, Flags& f) {
      if constexpr (RFL) {
        const __amdgpu_buffer_rsrc_t rt = chunk_rs(p.term, c, 1), rr = chunk_rs(p.trunc, c, 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t off = (uint32_t)((int64_t)(4 * fword(i) + m) * E + scol);
            f[i][0][m] = __builtin_amdgcn_raw_buffer_load_b32(rt, off, 0, 2);
            f[i][1][m] = __builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, 2);
          }
      }
    };
    auto write_flags = [&](int c, const Flags& f) {
      if constexpr (RFL) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint32_t w4[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) w4[m] = bytes_nonzero(f[i][0][m]) | (bytes_nonzero(f[i][1][m]) << 1);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s_fw[c % 3][scol + j][fword(i)] = ((w4[0] >> (8 * j)) & 0xffu) | (((w4[1] >> (8 * j)) & 0xffu) << 8) |
                                              (((w4[2] >> (8 * j)) & 0xffu) << 16) |
                                              (((w4[3] >> (8 * j)) & 0xffu) << 24);
        }
      }
    };
    Flags f0, f1;
    issue_flags(0, f0);
    issue_flags(1, f1);
    write_flags(0, f0);
    issue_flags(2, f0);
    write_flags(1, f1);
    issue_flags(3, f1);
    lds_done();
    tick_barrier();  // the prologue's two (chunks 0 and 1's flags written before the first)
    tick_barrier();
    // tick s: chunk s-1's outputs stored, chunk s+2's flags written (set s % 2)
    // and chunk s+4's requested into that set
    auto tick = [&](int s, Flags& f) {
      store_out(s - 1);
      write_flags(s + 2, f);
      issue_flags(s + 4, f);
      lds_done();
      tick_barrier();
    };
    for (int s = 0; s < ticks; s += 2) {
      tick(s, f0);
      if (s + 1 < ticks) tick(s + 1, f1);
    }
    store_out(ticks - 1);
  } else if (wave >= NC) {
    // ================================================================ DMA
    const int dw = wave - NC;
    const float* srcs[5] = {p.r, p.v, p.aux, p.pi, p.mu};
    // requests of tick t: flags of chunk t + NFL, streams of chunk t + NSL - 2
    auto issue = [&](int t) {
      if constexpr (DMAF) {
        const int c = t + NFL;  // >= 0
#pragma unroll
        for (int i = 0; i < 2 * NQF / ND; ++i) {
          const int idx = dw + ND * i, a = idx / NQF, q = idx % NQF;
          const uint32_t off = (uint32_t)((int64_t)(q * SPF + lane / LPF) * E + (lane % LPF) * 16);
          const __amdgpu_buffer_rsrc_t rs = chunk_rs(a ? p.trunc : p.term, c, 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)&s_f[c % NFL][a][q][0], 16, off, 0, 0, 0);
        }
      }
      const int c = t + NSL - 2;
      if (c < 0) return;  // (the prologue's first tick: flags only)
#pragma unroll
      for (int i = 0; i < NS * NQ / ND; ++i) {
        const int idx = dw + ND * i, st = idx / NQ, q = idx % NQ;
        // (arguments in variables: with a call in the builtin's argument list
        // the host pass drops the kernel's stub)
        const __amdgpu_buffer_rsrc_t rs = chunk_rs(srcs[st], c, ES);
        const uint32_t off = data_off(q);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)&s_d[c % NSL][st][q][0], 16, off, 0, 0, 0);
      }
    };
    // before the first tick: chunk 0's flags landed (first barrier), then chunk
    // 0's streams and chunk 1's flags (second)
    for (int t = 1 - NSL; t < 0; ++t) issue(t);
    wait_vmcnt<WAIT0>();
    tick_barrier();
    wait_vmcnt<WAITN>();
    tick_barrier();
    for (int s = 0; s < ticks; ++s) {
      issue(s);
      wait_vmcnt<WAITN>();  // chunk s+1's streams and chunk s+2's flags landed
      tick_barrier();
    }
    wait_vmcnt<0>();  // no DMA into this block's LDS may outlive the block
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
    constexpr bool FAST = Tr::kRetrace || !__is_same(S, F32S);
    // the lane's 4 steps lie in one group of every array
    const int dq = (int)cs_local / SPI, dr = (int)cs_local % SPI;
    const int fq = (int)cs_local / SPF, fr = (int)cs_local % SPF;

    int col[2];
    float rowv[2];
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

    struct Side {
      unsigned tb[2], rb[2];
      float boot[2][K];
    };
    // flags of chunk s from LDS (none past the last chunk), and its
    // bootstraps requested (lanes and steps without one pass an offset
    // outside the resource)
    auto side_of = [&](int s, Side& o) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        o.tb[it] = o.rb[it] = 0u;
#pragma unroll
        for (int m = 0; m < K; ++m) o.boot[it][m] = 0.0f;
      }
      if constexpr (RFL) {
        if (s < ticks) {
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const uint32_t w = s_fw[s % 3][col[it]][cs_local / 4];
            o.tb[it] = ((w & 1u) | ((w >> 7) & 2u) | ((w >> 14) & 4u) | ((w >> 21) & 8u)) & tmask;
            o.rb[it] = (((w >> 1) & 1u) | ((w >> 8) & 2u) | ((w >> 15) & 4u) | ((w >> 22) & 8u)) & rmask;
          }
        }
      }
      if constexpr (DMAF) {
        if (s < ticks) {
          const int fs = s % NFL;
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            unsigned tb = 0u, rb = 0u;
#pragma unroll
            for (int m = 0; m < K; ++m) {
              const int at = (fr + m) * EB + col[it];
              tb |= (s_f[fs][0][fq][at] != 0 ? 1u : 0u) << m;
              rb |= (s_f[fs][1][fq][at] != 0 ? 1u : 0u) << m;
            }
            o.tb[it] = tb & tmask;
            o.rb[it] = rb & rmask;
          }
        }
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
    auto cell = [&](int slot, int st, int it, int m) -> unsigned char* {
      return &s_d[slot][st][dq][(dr + m) * RB + col[it] * ES];
    };
    auto tick = [&](int s, const Side& cur, Side& nxt) {
      side_of(s + 1, nxt);
      const int slot = s % NSL;
      const int64_t t0 = (REV ? (int64_t)(ticks - 1 - s) : (int64_t)s) * SPAN;
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        LaneIn<Est, K> d;
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int m = 0; m < K; ++m) {
            if constexpr (ES == 4) d.s[st][m] = *reinterpret_cast<const float*>(cell(slot, st, it, m));
            else d.s[st][m] = s_to_f32<S>(*reinterpret_cast<const uint16_t*>(cell(slot, st, it, m)));
          }
#pragma unroll
        for (int m = 0; m < K; ++m) d.tb[m] = cur.boot[it][m];
        d.rowv = rowv[it];
        float o[2][K];
        stream_tile<Est, L, K, true, FAST, true>(d, sc, cur.tb[it], cur.rb[it], (uint32_t)t0 + cs_local, T,
                                                 team_first_lane, lane, C[it], carry[it], o[0], o[1]);
#pragma unroll
        for (int oi = 0; oi < NOUT; ++oi)
#pragma unroll
          for (int m = 0; m < K; ++m) {
            if constexpr (ES == 4) *reinterpret_cast<float*>(cell(slot, oi, it, m)) = o[oi][m];
            else *reinterpret_cast<uint16_t*>(cell(slot, oi, it, m)) = f32_to_s<S>(o[oi][m]);
          }
      }
      lds_done();
      tick_barrier();
    };

    Side sa, sb;
    tick_barrier();  // chunk 0's flags are in LDS
    side_of(0, sa);
    lds_done();
    tick_barrier();  // chunk 0's streams and chunk 1's flags are in LDS; chunk 0's flag slot free
    tick(0, sa, sb);
    for (int s = 1; s < ticks; s += 2) {
      tick(s, sb, sa);
      if (s + 1 < ticks) tick(s + 1, sa, sb);
    }
  }
}

}  // namespace rlscan
