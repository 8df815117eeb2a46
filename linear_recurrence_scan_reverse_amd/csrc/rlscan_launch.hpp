// rlscan_launch.hpp -- host-side launch of the scan kernels: resolves optional
// inputs, routes a call to one of the kernels (streaming, pipelined with a
// persistent grid or one item per team, segmented for long rows, time-major),
// picks its team shape, sizes its grid
// and launches it on the caller's stream (one kernel; three for the
// segmented path).
#pragma once

#include <atomic>

#include "rlscan_duo.hpp"
#include "rlscan_kernel.hpp"
#include "rlscan_plan.hpp"
#include "rlscan_segment.hpp"
#include "rlscan_stream.hpp"
#include "rlscan_timemajor.hpp"
#include "rlscan_tmitem.hpp"
#include "rlscan_tmdma.hpp"

namespace rlscan {

struct LaunchShape {
  int L, K, W;       // lanes per team (W == 1), steps per lane per tile, waves per row
  bool one = false;  // one item per team (a grid covering every row group)
};

// Team shape by row length.  Short rows share a wave (16 or 32 lanes each) so
// that every lane still owns a 4-step chunk; rows up to 256 steps are one
// wave; longer rows use 2 or 4 waves whose totals meet in LDS, and rows
// beyond one tile loop over tiles with the carry in registers.
inline LaunchShape pick_shape(int64_t T) {
  if (T <= 16) return {16, 1, 1};
  if (T <= 32) return {16, 2, 1};
  if (T <= 64) return {16, 4, 1};
  if (T <= 128) return {32, 4, 1};
  if (T <= 256) return {64, 4, 1};
  if (T <= 512) return {64, 4, 2};
  return {64, 4, 4};
}

// Team shape for 16-bit storage: rows of 65 to 512 steps take 8 steps per
// lane (one 16-byte access per lane and stream, as 4 float32 steps are), so
// half as many lanes per row.  Measured at 16384 x 256 (bfloat16): TD(lambda)
// and GAE 13.0 -> 11.7 us, traces and prefix sums 10.1 -> 9.5 us, discounted
// returns 11.0 -> 10.5 us (with 4 blocks per CU: its usual 8 do not fit at 8
// steps per lane; 65536 x 256: 32.0 -> 28.6 us); V-trace unchanged and Retrace
// 17.4 -> 18.1 us, so those two keep 4 steps per lane -- except V-trace in the
// one-item form (one: the call takes it), where 8 measured faster at
// 16384 x 256 (bfloat16 15.3 -> 14.8 us; Retrace there 15.4 -> 16.4 us).
template <class Est>
inline LaunchShape pick_shape_16(int64_t T, bool one) {
  if (__is_same(Est, Retrace) || (__is_same(Est, Vtrace) && !one)) return pick_shape(T);
  if (T <= 64) return pick_shape(T);
  if (T <= 128) return {16, 8, 1};
  if (T <= 256) return {32, 8, 1};
  if (T <= 512) return {64, 8, 1};
  return pick_shape(T);
}

// Resident blocks per CU the persistent grid aims for (discounted returns, the
// lightest kernel, measured faster with more waves in flight: 11.4 vs 11.9 us
// at 16384 x 256; at 8 steps per lane its registers allow only 4).
template <class Est>
inline int blocks_per_cu(const LaunchShape& sh) { return (__is_same(Est, DiscountedReturn) && sh.K != 8) ? 8 : 4; }

// Estimators with a one-item-per-team form of the pipelined kernel (see
// prefer_oneshot).
template <class Est>
constexpr bool kOneShotEst = __is_same(Est, Retrace) || __is_same(Est, Vtrace) || __is_same(Est, DiscountedReturn) ||
                             __is_same(Est, TdLambda) || __is_same(Est, Gae) || __is_same(Est, EligibilityTrace) ||
                             __is_same(Est, EpisodicPrefixSum);

// Whether a call takes the pipelined kernel with one item per team: a grid
// that holds a team for every row group, each team loading its row's flags
// and inputs at once and exiting after one store, instead of the persistent
// grid that prefetches a team's next item (or the streaming kernel).  Without
// flag arrays (16384 x 256: Retrace 22.6 -> 19.0 us, V-trace 20.0 -> 17.9 us;
// 4096 x 256: 9.3 -> 6.8 and 7.5 -> 6.7 us) and with them, measured over
// E in {4096, 16384, 65536} x T in {64 .. 1024} against the routing below:
// Retrace faster at every point (16384 x 256: 22.6 -> 20.6 us; 4096 x 256:
// 11.4 -> 7.5 us; 2048 x 1024: 13.4 -> 12.1 us), V-trace faster up to 512
// steps (16384 x 256: 19.9 -> 19.1 us; 8192 x 128: 9.3 -> 7.3 us) but not at
// 1024 (4096 x 1024: 20.5 -> 21.3 us).  With 16-bit storage (bfloat16, same
// grid) Retrace again gained at every point (4096 x 256: 10.5 -> 6.6 us;
// 65536 x 256: 61.1 -> 56.1 us) and V-trace up to 256 steps (65536 x 256:
// 56.6 -> 51.8 us) but lost from 512 (16384 x 512: 29.6 -> 31.2 us).  In
// float32 the five lighter estimators ran slower or no faster than on the
// streaming kernel.  In 16-bit storage (where they run on the persistent
// pipelined kernel, not the streaming one; bfloat16 grid over E in
// {4096, 16384, 65536} x T in {64 .. 512}) TD(lambda) and GAE gained at every
// point but 4096 x 64 (16384 x 128: 10.2 -> 6.9 us; 4096 x 512: 11.9 ->
// 7.3 us; 65536 x 256: 32.7 -> 28.8 us), and discounted returns gained only
// with rows of 257 to 512 steps (4096 x 512: 11.0 -> 7.3 us; 16384 x 512:
// 17.2 -> 14.9 us; 4096 x 256: 7.2 -> 9.3 us).  The 16-bit eligibility traces
// and prefix sums, against the streaming kernel, gained from 16384 rows up
// (65536 x 256: 26.3 -> 21.1 us; 16384 x 512: 14.6 -> 12.8 us) and lost
// 0.3 us at 4096 x 64.  Rows up to 1024 steps are one tile of one team.
// esize: bytes per stored value.
template <class Est>
inline bool prefer_oneshot(const KernelArgs& a, int esize) {
  if constexpr (!kOneShotEst<Est>) {
    return false;
  } else {
    if constexpr (__is_same(Est, Retrace)) return a.T <= 1024;
    if constexpr (__is_same(Est, Vtrace)) return a.T <= (esize == 4 ? 512 : 256);
    if (esize != 2) return false;
    if constexpr (__is_same(Est, DiscountedReturn)) return a.T > 256 && a.T <= 512;
    return a.T <= 512;  // TD(lambda), GAE, eligibility traces, prefix sums
  }
}

// Rows a team scans per work item: one on this path (the kernel keeps the
// count as a template parameter, R).
template <class Est, int K>
constexpr int rows_per_item() { return 1; }

// The vector path needs whole tiles (T % span == 0) and every dense array base
// aligned to its K-element chunk.
inline bool vector_ok(const KernelArgs& a, int K, int span, int esize = 4) {
  if (a.T % span != 0) return false;
  const uintptr_t fa = (uintptr_t)(esize * K), ba = (uintptr_t)K;
  const float* fl[] = {a.r, a.v, a.aux, a.pi, a.mu, a.tboot, a.out0, a.out1};
  for (const float* q : fl)
    if (q && ((uintptr_t)q % fa) != 0) return false;
  const uint8_t* bl[] = {a.term, a.trunc};
  for (const uint8_t* q : bl)
    if (q && ((uintptr_t)q % ba) != 0) return false;
  return true;
}

// Replace absent optional inputs by valid stand-in addresses so the kernel's
// loads never branch; the has_* switches tell the kernel to ignore them.
inline KernelArgs resolve_optional(KernelArgs a) {
  a.has_term = a.term != nullptr;
  a.has_trunc = a.trunc != nullptr;
  if (!a.term) a.term = a.trunc;
  if (!a.trunc) a.trunc = a.term;
  a.has_row = a.row != nullptr;
  if (!a.row) a.row = a.r;  // [E,T] with T >= 1 holds at least E floats
  a.has_tboot = a.tboot != nullptr;
  if (!a.tboot) a.tboot = a.r;
  return a;
}

// Compute units of the current device, queried once per device (grids are
// sized from it on every call).
inline int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <class Est, int L, int K, int W, bool VEC, int OPT, class S = F32S>
inline hipError_t launch_one(const KernelArgs& a, hipStream_t s, const LaunchShape& sh) {
  constexpr int BLOCK = BlockShape<W>::kThreads;
  constexpr int TEAMS = BLOCK / ((W > 1) ? 64 * W : L);
  constexpr int R = rows_per_item<Est, K>();
  const int64_t groups = (a.E + R - 1) / R;
  int64_t blocks = (groups + TEAMS - 1) / TEAMS;
  KernelArgs arg = a;
  void* params[] = {&arg};
  if constexpr (kOneShotEst<Est>) {
    // the one-item grid is not capped: past 2^31 work-items (e.g. 2^27 rows of
    // 64 steps) the persistent grid below takes the call
    if (sh.one && blocks * BLOCK < (int64_t(1) << 31))
      return hipLaunchKernel(reinterpret_cast<const void*>(&scan_kernel<Est, L, K, W, R, VEC, OPT, S, true>),
                             dim3((unsigned)blocks), dim3(BLOCK), params, 0, s);
  }
  const int64_t resident = (int64_t)cu_count() * blocks_per_cu<Est>(sh);
  if (blocks > resident) blocks = resident;
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_kernel<Est, L, K, W, R, VEC, OPT, S>),
                         dim3((unsigned)blocks), dim3(BLOCK), params, 0, s);
}

template <class Est, int L, int K, int W, int OPT, class S = F32S>
inline hipError_t launch_vec(const KernelArgs& a, hipStream_t s, const LaunchShape& sh) {
  constexpr int SPAN = ((W > 1) ? 64 * W : L) * K;
  return vector_ok(a, K, SPAN, (int)sizeof(typename S::T)) ? launch_one<Est, L, K, W, true, OPT, S>(a, s, sh)
                                                           : launch_one<Est, L, K, W, false, OPT, S>(a, s, sh);
}

// OPT bit 0: a flag array is present; bit 1: the second output is written.
template <class Est, int L, int K, int W, class S = F32S>
inline hipError_t launch_shape(const KernelArgs& a, hipStream_t s, const LaunchShape& sh) {
  using Tr = Traits<Est>;
  const bool flags = a.has_term || a.has_trunc;
  if constexpr (Tr::kHasOut1) {
    const bool out1 = a.out1 != nullptr;
    if (flags) return out1 ? launch_vec<Est, L, K, W, 3, S>(a, s, sh) : launch_vec<Est, L, K, W, 1, S>(a, s, sh);
    return out1 ? launch_vec<Est, L, K, W, 2, S>(a, s, sh) : launch_vec<Est, L, K, W, 0, S>(a, s, sh);
  } else if constexpr (Tr::kUsesFlags) {
    return flags ? launch_vec<Est, L, K, W, 1, S>(a, s, sh) : launch_vec<Est, L, K, W, 0, S>(a, s, sh);
  } else {
    return launch_vec<Est, L, K, W, 0, S>(a, s, sh);
  }
}

// ----------------------------------------------------------------- streaming path
// Data lead (ticks) and blocks per CU of the streaming kernel (a sweep over
// leads 2..4 and 2..6 blocks per CU at 16384 x 256 favoured 2 and 2).
template <class Est>
constexpr int stream_lead() { return 2; }
constexpr int kStreamBlocksPerCu = 2;

template <class Est, int L, int OPT, class Fmt = F32S>
inline hipError_t launch_stream_one(const KernelArgs& a, hipStream_t s) {
  constexpr int P = stream_lead<Est>();
  constexpr int BPC = kStreamBlocksPerCu;
  using Cfg = StreamCfg<Est, (OPT & 1) != 0, P, BPC, Fmt>;
  constexpr int G = 64 / L;
  const int64_t nrg = (a.E + G - 1) / G;
  const int64_t cap = (int64_t)cu_count() * BPC;
  const int64_t per_wave = (nrg + Cfg::NC * cap - 1) / (Cfg::NC * cap);
  int64_t blocks = (nrg + Cfg::NC * per_wave - 1) / (Cfg::NC * per_wave);
  if (blocks < 1) blocks = 1;
  KernelArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&stream_kernel<Est, L, OPT, P, BPC, Fmt>),
                         dim3((unsigned)blocks), dim3(Cfg::kThreads), params, 0, s);
}

template <class Est, int L, class Fmt = F32S>
inline hipError_t launch_stream(const KernelArgs& a, hipStream_t s) {
  using Tr = Traits<Est>;
  const bool flags = a.has_term || a.has_trunc;
  if constexpr (Tr::kHasOut1) {
    const bool out1 = a.out1 != nullptr;
    if (flags) return out1 ? launch_stream_one<Est, L, 3, Fmt>(a, s) : launch_stream_one<Est, L, 1, Fmt>(a, s);
    return out1 ? launch_stream_one<Est, L, 2, Fmt>(a, s) : launch_stream_one<Est, L, 0, Fmt>(a, s);
  } else if constexpr (Tr::kUsesFlags) {
    return flags ? launch_stream_one<Est, L, 1, Fmt>(a, s) : launch_stream_one<Est, L, 0, Fmt>(a, s);
  } else {
    return launch_stream_one<Est, L, 0, Fmt>(a, s);
  }
}

// The streaming kernel takes rows made of whole tiles with every dense array
// 16-byte aligned (a lane moves 16 bytes per DMA); for 16-bit formats the
// row-value array must be 4-byte aligned and E even (row values travel as the
// aligned word holding them).
template <class Fmt = F32S>
inline int stream_team(const KernelArgs& a) {
  constexpr int ES = (int)sizeof(typename Fmt::T);
  int L = 0;
  if (a.T == 64) L = 16;
  else if (a.T == 128) L = 32;
  else if (a.T % 256 == 0) L = 64;
  if (L == 0 || !vector_ok(a, 16 / ES, L * 4, ES)) return 0;
  // flag bytes are fetched 16 at a time
  if ((uintptr_t)a.term % 16 != 0 || (uintptr_t)a.trunc % 16 != 0) return 0;
  if (ES == 2 && ((uintptr_t)a.row % 4 != 0 || a.E % 2 != 0)) return 0;
  return L;
}

// Whether the streaming kernel should take a call its rows allow (team width
// L).  Measured over E in {256 .. 16384} x T in {64 .. 4096}:
//  * a streaming compute wave walks the tiles of its rows one per tick, so
//    rows of 8 or more tiles, with fewer than two rows per compute wave the
//    grid can hold, run faster on the pipelined kernel, whose 4-wave teams
//    split a long row (up to 2.3x at 256 x 4096);
//  * V-trace with rows of more than one tile, and Retrace with flags
//    present, run faster pipelined at every size measured from 4096 rows up
//    (the per-wave bootstrap gather and the heavier per-step arithmetic
//    overlap better there than in ticks);
//  * discounted returns with flags stream faster up to 16384 rows (16384 x
//    256: 11.5 vs 12.4 us; 4096 x 1024: 11.9 vs 13.5 us) but not at 65536 rows
//    (65536 x 64: 12.6 vs 11.1 us).
template <class Est>
inline bool prefer_stream(const KernelArgs& a, int L) {
  const bool flags = a.has_term || a.has_trunc;
  if (__is_same(Est, Retrace) && flags) return false;
  if (__is_same(Est, DiscountedReturn) && flags && a.E > 32768) return false;
  if (__is_same(Est, Vtrace) && a.T > 256) return false;
  const int64_t ntiles = a.T / (4 * L);
  if (ntiles >= 8) {
    constexpr int P = stream_lead<Est>();
    constexpr int BPC = kStreamBlocksPerCu;
    const int nc = flags ? StreamCfg<Est, true, P, BPC>::NC : StreamCfg<Est, false, P, BPC>::NC;
    const int64_t nrg = (a.E + (64 / L) - 1) / (64 / L);
    if (nrg < 2 * (int64_t)cu_count() * BPC * nc) return false;
  }
  return true;
}

// ----------------------------------------------------------------- items of 1 KiB per array
// Rows of 64, 128 or 256 float32 steps (128, 256 or 512 16-bit steps) with
// every dense array 16-byte aligned (and the flag arrays K-byte aligned) can
// take a kernel whose items are 1 KiB of every array (whole rows): duo_kernel
// (two items per wave, the second staged through LDS), duo_reg_kernel (two
// items per wave, both in registers, each scanned as soon as its own loads
// land) or multi_reg_kernel with four items per wave (a software pipeline
// keeping two items ahead in flight).
enum DuoForm { kDuoNone = 0, kDuoLds = 1, kDuoReg = 2, kDuoReg4 = 4, kDuoLds4 = 5 };

// Float32 routing, from A/B runs on one MI355X with flags present (each form
// forced for every estimator, two interleaved rounds over E in {4096, 16384,
// 32768, 65536} x T in {64, 128, 256}; us, against the streaming or one-item
// pipelined kernel the call takes otherwise):
//  * discounted returns: two in registers everywhere (16384 x 64: 5.9 -> 4.5;
//    16384 x 256: 11.0 -> 9.4; 32768 x 256: 19.7 -> 16.2);
//  * TD(lambda), GAE: two in registers (16384 x 64: 5.9 -> 4.8; 16384 x 128:
//    8.1 -> 7.2; 65536 x 128: 22.4 -> 20.8), four at 16384 x 256 (12.0 ->
//    11.7);
//  * V-trace: four at 16384-32768 rows of 128 or 256 steps and 65536 x 64
//    (16384 x 256: 18.8 -> 18.1; 16384 x 128: 11.4 -> 10.2; 65536 x 64:
//    18.9 -> 17.8), two in registers at 32768 x 64, 65536 x 128 and 4096 x
//    256, LDS from 32768 rows of 256 steps (33.5 -> 31.7);
//  * Retrace: two in registers up to 16384 rows of 64 and up to 4096 rows
//    (4096 x 128: 5.5 -> 4.4), four at 32768 rows of 64 and 16384-32768 rows
//    of 128 (16384 x 128: 11.9 -> 10.8), LDS at 65536 x 128 and 16384-32768
//    rows of 256 (16384 x 256: 20.2 -> 19.6), there with four of item B's
//    five streams in LDS up to 16384 rows (three interleaved rounds: 19.72 ->
//    19.50; at 32768 x 256 four were 34.9-37.3 against 35.2 and stay three);
//  * traces and prefix sums: LDS for rows of 64 steps up to 16384 rows
//    (16384 x 64: 4.3 -> 4.0) and at 65536 x 256 (an earlier sweep: 32.2 ->
//    26.4), two in registers up to 4096 rows and at 16384 x 128 and 32768 x
//    64 (5.7 -> 5.4), the streaming kernel elsewhere (16384 x 256: 8.6 against
//    8.7 in registers).
// Row counts between the measured ones take the form of the next smaller one.
template <class Est>
inline int duo_form(const KernelArgs& a) {
  if (a.T != 64 && a.T != 128 && a.T != 256) return kDuoNone;
  const int L = (int)(a.T / 4);
  const int64_t items = (a.E + (64 / L) - 1) / (64 / L);
  if ((items + 7) / 8 * 256 > kMaxWorkItems) return kDuoNone;
  if (!vector_ok(a, 4, (int)a.T)) return kDuoNone;
  const int64_t E = a.E, T = a.T;
  if constexpr (__is_same(Est, DiscountedReturn)) return kDuoReg;
  if constexpr (__is_same(Est, TdLambda) || __is_same(Est, Gae))
    return (T == 256 && E >= 16384 && E < 32768) ? kDuoReg4 : kDuoReg;
  if constexpr (__is_same(Est, Vtrace)) {
    if (T == 64) return E >= 65536 ? kDuoReg4 : E >= 32768 ? kDuoReg : kDuoNone;
    if (T == 128) return E >= 65536 ? kDuoReg : E >= 16384 ? kDuoReg4 : kDuoNone;
    return E >= 32768 ? kDuoLds : E >= 16384 ? kDuoReg4 : E >= 4096 ? kDuoReg : kDuoNone;
  }
  if constexpr (__is_same(Est, Retrace)) {
    if (T == 64) return E >= 32768 ? kDuoReg4 : kDuoReg;
    if (T == 128) return E >= 65536 ? kDuoLds : E >= 16384 ? kDuoReg4 : E <= 4096 ? kDuoReg : kDuoNone;
    return E > 32768 ? kDuoNone : E > 16384 ? kDuoLds : E > 4096 ? kDuoLds4 : kDuoReg;
  }
  if constexpr (__is_same(Est, EligibilityTrace) || __is_same(Est, EpisodicPrefixSum)) {
    if ((T == 256 && E >= 65536) || (T == 64 && E <= 16384)) return kDuoLds;
    return (E <= 4096 || (T == 128 && E <= 16384) || (T == 64 && E <= 32768)) ? kDuoReg : kDuoNone;
  }
  return kDuoNone;
}

// 16-bit storage: two items per wave in registers, a lane holding 16 bytes of
// each array (8 steps; rows of 128, 256 or 512 steps, team width T / 8) or 8
// bytes (4 steps; rows of 64, 128 or 256, team width T / 4).  From bfloat16
// A/B runs over E in {4096, 16384, 32768, 65536} x T in {64 .. 512} against
// the kernels the calls took before (us):
//  * 16 bytes per lane: everywhere but V-trace at 4096 x 128 and traces /
//    prefix sums at 4096 x 256 (16384 x 256: discounted returns 10.6 -> 8.0,
//    TD(lambda) 10.1 -> 8.7, V-trace 14.5 -> 12.2, Retrace 14.8 -> 12.8,
//    traces 8.1 -> 6.7); the LDS form was 0.2-1.9 us slower at 16384 x 256,
//    four items per wave slower at most shapes;
//  * 8 bytes per lane, where it beat that: rows of 64 steps from 16384 rows
//    (TD(lambda) 32768 x 64: 6.7 -> 5.8; Retrace 65536 x 64: 14.8 -> 12.7),
//    rows of 128 up to 4096 rows (Retrace 5.0 -> 4.3; discounted returns
//    6.2 -> 4.4), and discounted returns, traces and prefix sums with rows
//    of 256 up to 4096 rows (4.7 -> 4.2); slower with 256 steps from 16384
//    rows (TD(lambda) 8.8 -> 9.6);
//  * four items per wave as a software pipeline (multi_reg_kernel) for rows
//    of 512 steps from 16384 rows: traces and prefix sums (16384 x 512: 11.4
//    -> 10.1; 32768 x 512: 19.5 -> 18.0), TD(lambda) and GAE below 32768
//    rows (16384 x 512: 15.2 -> 14.2; even at 32768) -- the rows of the
//    float32 rule for TD(lambda) and GAE, at half the bytes per step; at
//    256 steps and below it was even or slower (TD(lambda) 4096 x 256: 4.7
//    -> 6.0).
struct Duo16 {
  int L;     // team width (0: not taken)
  int lb;    // bytes per lane and array
  int form;  // kDuoReg or kDuoReg4
};
template <class Est>
inline Duo16 duo_form_16(const KernelArgs& a) {
  const int64_t E = a.E, T = a.T;
  constexpr bool light = __is_same(Est, DiscountedReturn) || __is_same(Est, EligibilityTrace) ||
                         __is_same(Est, EpisodicPrefixSum);
  int lb = 16;
  if ((T == 64 && E >= 16384) || (T == 128 && E <= 4096) || (T == 256 && E <= 4096 && light)) lb = 8;
  else if (T != 128 && T != 256 && T != 512) return Duo16{0, 0, 0};
  const int L = (int)(T * 2 / lb);
  const int64_t items = (E + (64 / L) - 1) / (64 / L);
  if ((items + 7) / 8 * 256 > kMaxWorkItems) return Duo16{0, 0, 0};
  if (!vector_ok(a, lb / 2, (int)T, 2)) return Duo16{0, 0, 0};
  if (lb == 16 && (__is_same(Est, EligibilityTrace) || __is_same(Est, EpisodicPrefixSum)) && E <= 4096 && T == 256)
    return Duo16{0, 0, 0};
  constexpr bool fwd = __is_same(Est, EligibilityTrace) || __is_same(Est, EpisodicPrefixSum);
  constexpr bool td = __is_same(Est, TdLambda) || __is_same(Est, Gae);
  const bool four = T == 512 && E >= 16384 && (fwd || (td && E < 32768));
  return Duo16{L, lb, four ? kDuoReg4 : kDuoReg};
}

template <class Est, int L, int OPT, class S = F32S>
inline hipError_t launch_duo_opt(const KernelArgs& a, hipStream_t s, int form) {
  const int64_t items = (a.E + (64 / L) - 1) / (64 / L);
  KernelArgs arg = a;
  void* params[] = {&arg};
  const void* k = reinterpret_cast<const void*>(&duo_reg_kernel<Est, L, OPT, S>);
  if constexpr (!__is_same(S, F32S)) {
    if (a.T == 4 * L) k = reinterpret_cast<const void*>(&duo_reg_kernel<Est, L, OPT, S, 8>);  // 8 bytes per lane
  }
  int per_block = 8;  // items per block of 4 waves
  if constexpr (__is_same(S, F32S)) {
    if (form == kDuoLds) k = reinterpret_cast<const void*>(&duo_kernel<Est, L, OPT>);
    if (form == kDuoLds4) k = reinterpret_cast<const void*>(&duo_kernel<Est, L, OPT, S, 4>);
  }
  if (form == kDuoReg4) {
    k = reinterpret_cast<const void*>(&multi_reg_kernel<Est, L, OPT, S, 4>);
    per_block = 16;
  }
  return hipLaunchKernel(k, dim3((unsigned)((items + per_block - 1) / per_block)), dim3(256), params, 0, s);
}

template <class Est, int L, class S = F32S>
inline hipError_t launch_duo(const KernelArgs& a, hipStream_t s, int form) {
  using Tr = Traits<Est>;
  const bool flags = a.has_term || a.has_trunc;
  if constexpr (Tr::kHasOut1) {
    const bool out1 = a.out1 != nullptr;
    if (flags) return out1 ? launch_duo_opt<Est, L, 3, S>(a, s, form) : launch_duo_opt<Est, L, 1, S>(a, s, form);
    return out1 ? launch_duo_opt<Est, L, 2, S>(a, s, form) : launch_duo_opt<Est, L, 0, S>(a, s, form);
  } else {
    return flags ? launch_duo_opt<Est, L, 1, S>(a, s, form) : launch_duo_opt<Est, L, 0, S>(a, s, form);
  }
}

// ----------------------------------------------------------------- segmented path
// Rows of at least kSegMinT steps, kSegMaxE rows or fewer, are cut into
// segments (row_segments) so that passes 1 and 3 run about 32 waves per CU;
// segments hold at least four tiles and the last one takes the remainder.
// Measured: 1 x 262144 steps 12-14x faster than whole rows, 16 x 65536 3-4x;
// at 256 rows whole-row teams already fill the GPU and win (the segmented
// path reads its inputs twice).
inline SegPlan segment_plan(const KernelArgs& a) { return row_segments(a.E, a.T, cu_count()); }

template <class Est, int OPT, class S = F32S>
inline hipError_t launch_segmented_opt(const KernelArgs& a, hipStream_t s, const SegPlan& plan) {
  int64_t seg_len = plan.len;
  int64_t nseg = plan.nseg;  // the last segment takes the remainder
  KernelArgs arg = a;
  void* params[] = {&arg, &seg_len, &nseg};
  const bool vec = vector_ok(a, 4, kSegTile, (int)sizeof(typename S::T));
  const dim3 block(256);
  const dim3 grid_seg((unsigned)((a.E * nseg + 3) / 4));
  const dim3 grid_row((unsigned)((a.E + 3) / 4));
  const void* agg = vec ? reinterpret_cast<const void*>(&seg_kernel<Est, true, true, OPT, S>)
                        : reinterpret_cast<const void*>(&seg_kernel<Est, true, false, OPT, S>);
  const void* apply = vec ? reinterpret_cast<const void*>(&seg_kernel<Est, false, true, OPT, S>)
                          : reinterpret_cast<const void*>(&seg_kernel<Est, false, false, OPT, S>);
  hipError_t e = hipLaunchKernel(agg, grid_seg, block, params, 0, s);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&seg_carry_kernel<Est, S>), grid_row, block, params, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(apply, grid_seg, block, params, 0, s);
}

template <class Est, class S = F32S>
inline hipError_t launch_segmented(const KernelArgs& a, hipStream_t s, const SegPlan& plan) {
  using Tr = Traits<Est>;
  const bool flags = a.has_term || a.has_trunc;
  if constexpr (Tr::kHasOut1) {
    const bool out1 = a.out1 != nullptr;
    if (flags)
      return out1 ? launch_segmented_opt<Est, 3, S>(a, s, plan) : launch_segmented_opt<Est, 1, S>(a, s, plan);
    return out1 ? launch_segmented_opt<Est, 2, S>(a, s, plan) : launch_segmented_opt<Est, 0, S>(a, s, plan);
  } else if constexpr (Tr::kUsesFlags) {
    return flags ? launch_segmented_opt<Est, 1, S>(a, s, plan) : launch_segmented_opt<Est, 0, S>(a, s, plan);
  } else {
    return launch_segmented_opt<Est, 0, S>(a, s, plan);
  }
}

template <class Est>
hipError_t launch(const KernelArgs& in, hipStream_t s) {
  const KernelArgs a = resolve_optional(in);
  if (const SegPlan plan = segment_plan(a); plan.len) return launch_segmented<Est>(a, s, plan);
  if constexpr (!Traits<Est>::kDual && !Traits<Est>::kLinear) {
    if (const int form = duo_form<Est>(a); form != kDuoNone) {
      switch (a.T) {
        case 64: return launch_duo<Est, 16>(a, s, form);
        case 128: return launch_duo<Est, 32>(a, s, form);
        default: return launch_duo<Est, 64>(a, s, form);
      }
    }
  }
  const bool one = prefer_oneshot<Est>(a, 4);
  const int team = one ? 0 : stream_team<F32S>(a);
  switch ((team != 0 && prefer_stream<Est>(a, team)) ? team : 0) {
    case 16: return launch_stream<Est, 16>(a, s);
    case 32: return launch_stream<Est, 32>(a, s);
    case 64: return launch_stream<Est, 64>(a, s);
    default: break;
  }
  LaunchShape sh = pick_shape(a.T);
  sh.one = one;
  switch (sh.W * 1000 + sh.L * 10 + sh.K) {
    case 1000 + 160 + 1: return launch_shape<Est, 16, 1, 1>(a, s, sh);
    case 1000 + 160 + 2: return launch_shape<Est, 16, 2, 1>(a, s, sh);
    case 1000 + 160 + 4: return launch_shape<Est, 16, 4, 1>(a, s, sh);
    case 1000 + 320 + 4: return launch_shape<Est, 32, 4, 1>(a, s, sh);
    case 1000 + 640 + 4: return launch_shape<Est, 64, 4, 1>(a, s, sh);
    case 2000 + 640 + 4: return launch_shape<Est, 64, 4, 2>(a, s, sh);
    case 4000 + 640 + 4: return launch_shape<Est, 64, 4, 4>(a, s, sh);
    default: return hipErrorInvalidConfiguration;
  }
}

// Values stored as 16-bit bf16 / fp16 (S = Bf16S, F16S): the segmented path
// for long rows; the two-item register kernel for rows of 128-512 steps
// (duo_form_16); the streaming kernel for traces and prefix sums where the
// rows allow it and the float32 routing rule prefers it; else the pipelined
// kernel.  At 16384 x 256 (bfloat16) the streaming kernel ran traces and
// prefix sums in 8.7-9.3 us against 9.6-9.9 pipelined, but the five backward
// estimators 0.5-1.9 us slower than pipelined: at this size a streaming block
// walks only four items after a fill of up to four ticks, so halving the
// bytes does not shorten it.
template <class Est, class S>
hipError_t launch_typed(const KernelArgs& in, hipStream_t s) {
  const KernelArgs a = resolve_optional(in);
  if (const SegPlan plan = segment_plan(a); plan.len) return launch_segmented<Est, S>(a, s, plan);
  if constexpr (!Traits<Est>::kDual && !Traits<Est>::kLinear) {
    const Duo16 f = duo_form_16<Est>(a);
    switch (f.L) {
      case 16: return launch_duo<Est, 16, S>(a, s, f.form);
      case 32: return launch_duo<Est, 32, S>(a, s, f.form);
      case 64: return launch_duo<Est, 64, S>(a, s, f.form);
      default: break;
    }
  }
  const bool one = prefer_oneshot<Est>(a, (int)sizeof(typename S::T));
  if constexpr (Traits<Est>::kForwardRl) {
    const int team = one ? 0 : stream_team<S>(a);
    switch ((team != 0 && prefer_stream<Est>(a, team)) ? team : 0) {
      case 16: return launch_stream<Est, 16, S>(a, s);
      case 32: return launch_stream<Est, 32, S>(a, s);
      case 64: return launch_stream<Est, 64, S>(a, s);
      default: break;
    }
  }
  LaunchShape sh = pick_shape_16<Est>(a.T, one);
  sh.one = one;
  switch (sh.W * 1000 + sh.L * 10 + sh.K) {
    case 1000 + 160 + 8: return launch_shape<Est, 16, 8, 1, S>(a, s, sh);
    case 1000 + 320 + 8: return launch_shape<Est, 32, 8, 1, S>(a, s, sh);
    case 1000 + 640 + 8: return launch_shape<Est, 64, 8, 1, S>(a, s, sh);
    case 1000 + 160 + 1: return launch_shape<Est, 16, 1, 1, S>(a, s, sh);
    case 1000 + 160 + 2: return launch_shape<Est, 16, 2, 1, S>(a, s, sh);
    case 1000 + 160 + 4: return launch_shape<Est, 16, 4, 1, S>(a, s, sh);
    case 1000 + 320 + 4: return launch_shape<Est, 32, 4, 1, S>(a, s, sh);
    case 1000 + 640 + 4: return launch_shape<Est, 64, 4, 1, S>(a, s, sh);
    case 2000 + 640 + 4: return launch_shape<Est, 64, 4, 2, S>(a, s, sh);
    case 4000 + 640 + 4: return launch_shape<Est, 64, 4, 4, S>(a, s, sh);
    default: return hipErrorInvalidConfiguration;
  }
}

// ----------------------------------------------------------------- time-major path
// [T, E] arrays: one block of W waves per 64 environments, K steps per wave
// chunk.  Blocks of 16 waves keep 16 waves per CU at 16384 environments.
// A block overlaps no loads with its compute, so fewer, longer super-tiles
// win: 16-step chunks (a 256-step row in one super-tile), except V-trace and
// Retrace, whose registers allow 8 (at 16384 x 256: TD(lambda) 17.5 -> 14.5
// us from 8 to 16 steps; 8 waves per block were slower everywhere).
template <class Est>
constexpr int tm_waves() { return 16; }
template <class Est>
constexpr int tm_chunk() { return Traits<Est>::kStreams >= 3 ? 8 : 16; }

// Few column groups and long columns: blocks of MODE 0 would leave most CUs
// idle and walk thousands of steps each, so time is cut into segments
// (tm_segments; see tm_kernel) giving about two blocks per CU, of at least 256
// steps and a multiple of 256 (whole super-tiles; the parked float64 pair
// needs at most 8 rows); the last segment takes the remainder.  At most
// kTmMaxSeg segments per column (the carry kernel's 16 waves x kTmCarrySeg).
// The item form of the time-major path (tm_item_kernel): one recurrence of
// at most three streams (or Retrace), whole 64-step chunks, 16-byte aligned
// per-step arrays, every storage format.  Blocks of 64 environments when there are at least as many
// such column groups as CUs, else of 32 (twice the blocks; with 32 at many
// environments the arrays streamed more slowly: 16384 x 256 discounted
// returns 12.5 us with 64, 16.4 with 32; 4096 x 256: 10.1 with 64, 8.9 with
// 32).  Routing, from a sweep of 1024 to 32768 environments and 64 to 2048
// steps (float32, one MI355X):
//  * at columns of exactly one super-tile of tm_kernel (256 steps, 128 for
//    V-trace), with 64-environment blocks, tm_kernel has every load of a
//    column in flight at once and the two are close; each estimator and
//    format takes the faster at 16384 and 32768 environments: V-trace and
//    16-bit traces and prefix sums stay with tm_kernel (V-trace 16384 x 128:
//    12.3 against 12.5 us; bfloat16 traces 16384 x 256: 8.7 against 9.5),
//    the others take the item form (32768 x 256: float32 discounted returns
//    22.1 -> 19.8, traces 19.2 -> 17.8; float32 TD(lambda) and GAE 16384 x
//    256, from its DMA form: 13.8 / 14.1 -> 13.5 / 13.4);
//  * a block walks its columns' chunks one after another, so long columns
//    over few blocks go to the segmented path: the item form takes columns of
//    up to 16 chunks, or any length with at least half as many blocks as CUs
//    (TD(lambda) 2048 x 2048: 31.1 us segmented, 47.5 item form; 4096 x 2048:
//    58.2 and 49.6; 4096 x 512: 26.4 and 15.6);
//  * Retrace's five streams fit in LDS only with 32-environment blocks; with
//    at least one 64-environment column group per CU tm_kernel stays faster
//    for it (16384 x 256: 25.4 us against 31.6), below that the item form
//    (4096 x 512: 41.8 -> 20.9 us, 8192 x 1024: 95.4 -> 53.3);
//  * everywhere else it was the faster one (float32 16384 x 320: TD(lambda)
//    23.6 -> 18.2 us, V-trace 34.2 -> 27.1; 16384 x 64: 11.0 -> 6.8;
//    bfloat16 32768 x 64 discounted returns 22.9 -> 8.3, 4096 x 512
//    TD(lambda) 32.0 -> 16.8).
template <class Est, class S>
constexpr bool tm_item_ok() {
  return !Traits<Est>::kDual && (Traits<Est>::kStreams <= 3 || Traits<Est>::kStreams == 5);
}
// environments per block of the item form, or 0 where the other kernels take the call
template <class Est, class S>
inline int tm_item_envs(const KernelArgs& a, int cus) {
  using Tr = Traits<Est>;
  auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  if (!al(a.r) || !al(a.v) || !al(a.aux) || !al(a.term) || !al(a.trunc) || !al(a.out0) || !al(a.out1))
    return 0;
  // one super-tile of tm_kernel: the faster kernel measured per estimator and format
  constexpr bool keep_tm = Tr::kStreams == 3 || (!__is_same(S, F32S) && !Tr::kBackwardRl);
  static_assert(kTiChunkSteps == kTiChunk, "one chunk size");
  return tm_item_block_envs(a.E, a.T, cus, Tr::kStreams, (int64_t)tm_waves<Est>() * tm_chunk<Est>(), keep_tm);
}

// Data slots of the DMA item form (tm_dma_kernel) for a kernel of 64-
// environment blocks: the most that fit, up to four, or 0 where three do not
// (V-trace's three float32 streams with flags, Retrace), which keep the
// register item form.  From A/B runs on one MI355X against the register form
// (us): bfloat16 16384 x 256 V-trace 20.2 -> 17.1, TD(lambda) 13.7 -> 12.5;
// float32 16384 x 512 TD(lambda) 24.9 -> 22.1, traces 17.7 -> 14.1; float32
// discounted returns and traces at 16384 x 256 even (11.0 / 9.5); six slots
// (more chunks in flight) were slower at every shape (16384 x 512 traces
// 16.2).  With 32-environment blocks (a CU then holds two blocks) it was
// slower (4096 x 256 traces 6.2 -> 7.3, 4096 x 512 discounted returns 11.8 ->
// 12.7) and they keep the register form, as do columns of fewer than four
// chunks (one chunk: float32 32768 x 64 traces 6.6 -> 8.2, its prologue
// exposed) and float32 discounted returns (32768 x 256: 19.8 -> 21.4; one
// stream, whose two chunks in registers already keep up).
constexpr int kTdMaxSlots = 4;
constexpr int64_t kTdMinSteps = 256;
template <class Est, int OPT, class S>
constexpr int td_slots() {
  if (__is_same(Est, DiscountedReturn) && __is_same(S, F32S)) return 0;
  constexpr bool flags = (OPT & 1) && Traits<Est>::kUsesFlags;
  for (int n = kTdMaxSlots; n >= 3; --n)
    if (td_fits(Traits<Est>::kStreams, 64, (int)sizeof(typename S::T), n, flags)) return n;
  return 0;
}

template <class Est, int OPT, class S>
inline hipError_t launch_tm_opt(const KernelArgs& a, hipStream_t s) {
  constexpr int W = tm_waves<Est>(), K = tm_chunk<Est>();
  static_assert(W == kTmWaves, "the grid limit assumes kTmWaves waves per block");
  const int64_t groups = (a.E + 63) / 64;
  const SegPlan plan = tm_segments(a.E, a.T, cu_count());
  int64_t seg_len = plan.len;
  int64_t nseg = plan.nseg;  // the last segment takes the remainder
  // grids of at most 2^32 - 1 work-items (the C ABI refuses larger shapes first)
  if (groups * nseg * 64 * W > kMaxWorkItems || nseg > kTmMaxSeg) return hipErrorInvalidConfiguration;
  KernelArgs arg = a;
  if constexpr (tm_item_ok<Est, S>()) {
    if (const int eb = tm_item_envs<Est, S>(a, cu_count())) {
      void* p1[] = {&arg};
      const dim3 grid((unsigned)(a.E / eb));
      constexpr int nsl = Traits<Est>::kStreams <= 3 ? td_slots<Est, OPT, S>() : 0;
      if constexpr (nsl != 0) {
        if (eb == 64 && a.T >= kTdMinSteps)
          return hipLaunchKernel(reinterpret_cast<const void*>(&tm_dma_kernel<Est, OPT, 64, S, nsl>), grid,
                                 dim3(td_threads<64>()), p1, 0, s);
      }
      // V-trace's three float32 streams with flags: the flags through the
      // storer waves' registers (three slots of one word per 4 steps, which
      // fit beside three data slots where the raw flag bytes do not); 16384 x
      // 256: 21.6 -> 17.9 us, 16384 x 512: 38.9 -> 35.6, 32768 x 256: 39.9 ->
      // 37.5 against the register item form
      constexpr bool rf = Traits<Est>::kStreams == 3 && nsl == 0 && (OPT & 1) && Traits<Est>::kUsesFlags &&
                          td_fits(3, 64, (int)sizeof(typename S::T), 3, true, true);
      if constexpr (rf) {
        if (eb == 64 && a.T >= kTdMinSteps)
          return hipLaunchKernel(reinterpret_cast<const void*>(&tm_dma_kernel<Est, OPT, 64, S, 3, true>), grid,
                                 dim3(td_threads<64>()), p1, 0, s);
      }
      if constexpr (Traits<Est>::kStreams <= 3) {
        if (eb == 64)
          return hipLaunchKernel(reinterpret_cast<const void*>(&tm_item_kernel<Est, OPT, 64, S>), grid,
                                 dim3(ti_threads<64>()), p1, 0, s);
      }
      return hipLaunchKernel(reinterpret_cast<const void*>(&tm_item_kernel<Est, OPT, 32, S>), grid,
                             dim3(ti_threads<32>()), p1, 0, s);
    }
  }
  void* params[] = {&arg, &seg_len, &nseg};
  const dim3 block(64 * W);
  if (nseg == 1)
    return hipLaunchKernel(reinterpret_cast<const void*>(&tm_kernel<Est, W, K, OPT, S, 0>), dim3((unsigned)groups),
                           block, params, 0, s);
  const dim3 grid((unsigned)(groups * nseg));
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&tm_kernel<Est, W, K, OPT, S, 1>), grid, block,
                                 params, 0, s);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&tm_carry_kernel<Est, S>), dim3((unsigned)groups), dim3(1024),
                      params, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&tm_kernel<Est, W, K, OPT, S, 2>), grid, block, params, 0, s);
}

template <class Est, class S = F32S>
hipError_t launch_tm(const KernelArgs& in, hipStream_t s) {
  using Tr = Traits<Est>;
  // one environment: [T, 1] is laid out as [1, T], so the row-major path
  // (whose long rows are split into segments) takes it
  if (in.E == 1) {
    if constexpr (__is_same(S, F32S)) return launch<Est>(in, s);
    else return launch_typed<Est, S>(in, s);
  }
  const KernelArgs a = resolve_optional(in);
  const bool flags = a.has_term || a.has_trunc;
  if constexpr (Tr::kHasOut1) {
    const bool out1 = a.out1 != nullptr;
    if (flags) return out1 ? launch_tm_opt<Est, 3, S>(a, s) : launch_tm_opt<Est, 1, S>(a, s);
    return out1 ? launch_tm_opt<Est, 2, S>(a, s) : launch_tm_opt<Est, 0, S>(a, s);
  } else {
    return flags ? launch_tm_opt<Est, 1, S>(a, s) : launch_tm_opt<Est, 0, S>(a, s);
  }
}

// Discounted returns (out0) and TD(lambda) returns (out1) of one rollout: one
// streaming pass where the rows allow it, else the two single-output kernels.
hipError_t launch_returns_td_lambda(const KernelArgs& in, hipStream_t s);

// Vector-valued eligibility traces over [E, T, D] (or [T, E, D]) features,
// one kernel; fmt: 0 float32, 1 bfloat16, 2 float16.
hipError_t launch_traces_vec(int fmt, bool time_major, const float* x, const uint8_t* term, const uint8_t* trunc,
                             const float* init, float* out, int64_t E, int64_t T, int64_t D, double gamma,
                             double lam, hipStream_t s);

// One translation unit per estimator instantiates launch<Est>.
extern template hipError_t launch<DiscountedReturn>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<TdLambda>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<Gae>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<Vtrace>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<Retrace>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<EligibilityTrace>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<EpisodicPrefixSum>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<LinearScanReverse>(const KernelArgs&, hipStream_t);
extern template hipError_t launch<LinearScanForward>(const KernelArgs&, hipStream_t);
#define RLSCAN_TYPED_EXTERN(EST)                                                       \
  extern template hipError_t launch_typed<EST, Bf16S>(const KernelArgs&, hipStream_t); \
  extern template hipError_t launch_typed<EST, F16S>(const KernelArgs&, hipStream_t);  \
  extern template hipError_t launch_tm<EST, F32S>(const KernelArgs&, hipStream_t);     \
  extern template hipError_t launch_tm<EST, Bf16S>(const KernelArgs&, hipStream_t);    \
  extern template hipError_t launch_tm<EST, F16S>(const KernelArgs&, hipStream_t);
RLSCAN_TYPED_EXTERN(DiscountedReturn)
RLSCAN_TYPED_EXTERN(TdLambda)
RLSCAN_TYPED_EXTERN(Gae)
RLSCAN_TYPED_EXTERN(Vtrace)
RLSCAN_TYPED_EXTERN(Retrace)
RLSCAN_TYPED_EXTERN(EligibilityTrace)
RLSCAN_TYPED_EXTERN(EpisodicPrefixSum)
RLSCAN_TYPED_EXTERN(LinearScanReverse)
RLSCAN_TYPED_EXTERN(LinearScanForward)
#undef RLSCAN_TYPED_EXTERN

}  // namespace rlscan
