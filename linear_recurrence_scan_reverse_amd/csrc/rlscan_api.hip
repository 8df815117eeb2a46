// rlscan_api.hip -- the C ABI of librlscan (declared in include/rlscan.h).
//
// Every entry point validates its arguments on the host before touching HIP,
// fills the kernel argument block and enqueues its kernels (one, or three for
// long rows with few rows) on the caller's stream.  Nothing is allocated and
// no state is kept.
#include <cmath>
#include <cstdint>

#include "rlscan.h"
#include "rlscan_launch.hpp"

namespace {

using rlscan::KernelArgs;

bool finite(float x) { return std::isfinite(x); }
bool in_unit(float x) { return finite(x) && x >= 0.0f && x <= 1.0f; }

// E, T >= 0, T below 2^30 (the kernels address a row with 32-bit byte
// offsets) and E*T*8 bytes representable (int64).
rlscan_status check_shape(int64_t E, int64_t T) {
  if (E < 0 || T < 0 || T >= RLSCAN_MAX_T) return RLSCAN_ERR_SHAPE;
  if (T > 0 && E > (INT64_MAX / 8) / T) return RLSCAN_ERR_SHAPE;
  return RLSCAN_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
  const uintptr_t b = (uintptr_t)p;
  return Range{b, b + (uintptr_t)bytes};
}

bool overlap(const Range& x, const Range& y) { return x.lo < y.hi && y.lo < x.hi; }

bool misaligned(const void* p, int esize = 4) { return p && ((uintptr_t)p % (uintptr_t)esize) != 0; }

// Bytes per stored value of a storage format (0: not a format).
int elem_size(rlscan_format f) {
  switch (f) {
    case RLSCAN_FORMAT_F32: return 4;
    case RLSCAN_FORMAT_BF16: return 2;
    case RLSCAN_FORMAT_F16: return 2;
  }
  return 0;
}

// Inputs and outputs of one call, for the NULL / alignment / overlap checks.
struct Io {
  const void* in[12];
  int64_t in_bytes[12];
  int n_in = 0;
  const void* out[2];
  int n_out = 0;
  void add_in(const void* p, int64_t bytes) {
    if (p) {
      in[n_in] = p;
      in_bytes[n_in] = bytes;
      ++n_in;
    }
  }
  void add_out(const void* p) {
    if (p) out[n_out++] = p;
  }
};

rlscan_status check_io(const Io& io, int64_t E, int64_t T, int esize = 4) {
  const int64_t obytes = esize * E * T;
  for (int i = 0; i < io.n_out; ++i) {
    if (misaligned(io.out[i], esize)) return RLSCAN_ERR_ALIGN;
    const Range ro = span(io.out[i], obytes);
    for (int j = 0; j < io.n_in; ++j)
      if (overlap(ro, span(io.in[j], io.in_bytes[j]))) return RLSCAN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(ro, span(io.out[j], obytes))) return RLSCAN_ERR_ALIAS;
  }
  return RLSCAN_OK;
}

rlscan_status launched(hipError_t e) { return e == hipSuccess ? RLSCAN_OK : RLSCAN_ERR_HIP; }

KernelArgs blank(int64_t E, int64_t T) {
  KernelArgs a{};
  a.E = E;
  a.T = T;
  return a;
}

// Shared validation for the five backward estimators: flags + bootstraps.
rlscan_status common_backward(Io& io, const uint8_t* term, const uint8_t* trunc, const void* boot,
                              const void* tboot, int64_t E, int64_t T, int esize = 4) {
  if (misaligned(boot, esize) || misaligned(tboot, esize)) return RLSCAN_ERR_ALIGN;
  io.add_in(term, E * T);
  io.add_in(trunc, E * T);
  io.add_in(boot, esize * E);
  io.add_in(tboot, esize * E * T);
  return RLSCAN_OK;
}

const float* fp(const void* p) { return static_cast<const float*>(p); }
float* fp(void* p) { return static_cast<float*>(p); }

bool layout_ok(rlscan_layout l) { return l == RLSCAN_LAYOUT_ENV_MAJOR || l == RLSCAN_LAYOUT_TIME_MAJOR; }

// Shapes whose grid would pass 2^32 - 1 work-items: time-major calls take one
// block of 16 waves per 64 environments (about 2^28 environments at most).
bool grid_fits(rlscan_layout l, int64_t E) { return l != RLSCAN_LAYOUT_TIME_MAJOR || rlscan::tm_grid_ok(E); }

// One estimator, one storage format, one layout.
template <class Est>
hipError_t launch_fmt(rlscan_format f, rlscan_layout l, const KernelArgs& a, hipStream_t s) {
  if (l == RLSCAN_LAYOUT_TIME_MAJOR) {
    switch (f) {
      case RLSCAN_FORMAT_BF16: return rlscan::launch_tm<Est, rlscan::Bf16S>(a, s);
      case RLSCAN_FORMAT_F16: return rlscan::launch_tm<Est, rlscan::F16S>(a, s);
      default: return rlscan::launch_tm<Est, rlscan::F32S>(a, s);
    }
  }
  switch (f) {
    case RLSCAN_FORMAT_BF16: return rlscan::launch_typed<Est, rlscan::Bf16S>(a, s);
    case RLSCAN_FORMAT_F16: return rlscan::launch_typed<Est, rlscan::F16S>(a, s);
    default: return rlscan::launch<Est>(a, s);
  }
}

// ---------------------------------------------------------------- the estimators
// Each takes its values in storage format f and its [E, T] arrays in layout l.
rlscan_status impl_discounted_returns(rlscan_format f, rlscan_layout l, const void* rewards, const uint8_t* terminated,
                                      const uint8_t* truncated, const void* bootstrap_value,
                                      const void* trunc_bootstrap, void* returns, int64_t E, int64_t T,
                                      float gamma, hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!rewards || !returns) return RLSCAN_ERR_NULL;
  if (misaligned(rewards, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, es * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T, es)) != RLSCAN_OK)
    return st;
  io.add_out(returns);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(rewards);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(bootstrap_value);
  a.tboot = fp(trunc_bootstrap);
  a.out0 = fp(returns);
  a.gamma = gamma;
  return launched(launch_fmt<rlscan::DiscountedReturn>(f, l, a, stream));
}

rlscan_status impl_td_lambda(rlscan_format f, rlscan_layout l, const void* rewards, const void* values, const uint8_t* terminated,
                             const uint8_t* truncated, const void* bootstrap_value, const void* trunc_bootstrap,
                             void* returns, int64_t E, int64_t T, float gamma, float lambda, hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!rewards || !values || !returns) return RLSCAN_ERR_NULL;
  if (misaligned(rewards, es) || misaligned(values, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, es * E * T);
  io.add_in(values, es * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T, es)) != RLSCAN_OK)
    return st;
  io.add_out(returns);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(rewards);
  a.v = fp(values);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(bootstrap_value);
  a.tboot = fp(trunc_bootstrap);
  a.out0 = fp(returns);
  a.gamma = gamma;
  a.lam = lambda;
  return launched(launch_fmt<rlscan::TdLambda>(f, l, a, stream));
}

// Discounted and TD(lambda) returns: one fused pass for float32 [E,T] rows the
// streaming kernel takes, else the two single-output calls in turn.
rlscan_status impl_returns_td_lambda(rlscan_format f, rlscan_layout l, const void* rewards, const void* values,
                                     const uint8_t* terminated, const uint8_t* truncated, const void* bootstrap_value,
                                     const void* trunc_bootstrap, void* returns, void* td_returns, int64_t E, int64_t T,
                                     float gamma, float lambda, hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!rewards || !values || !returns || !td_returns) return RLSCAN_ERR_NULL;
  if (misaligned(rewards, es) || misaligned(values, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, es * E * T);
  io.add_in(values, es * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T, es)) != RLSCAN_OK)
    return st;
  io.add_out(returns);
  io.add_out(td_returns);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(rewards);
  a.v = fp(values);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(bootstrap_value);
  a.tboot = fp(trunc_bootstrap);
  a.out0 = fp(returns);
  a.out1 = fp(td_returns);
  a.gamma = gamma;
  a.lam = lambda;
  if (f == RLSCAN_FORMAT_F32 && l == RLSCAN_LAYOUT_ENV_MAJOR) return launched(rlscan::launch_returns_td_lambda(a, stream));
  KernelArgs dr = a;
  dr.v = nullptr;
  dr.out1 = nullptr;
  const hipError_t e = launch_fmt<rlscan::DiscountedReturn>(f, l, dr, stream);
  if (e != hipSuccess) return launched(e);
  KernelArgs td = a;
  td.out0 = a.out1;
  td.out1 = nullptr;
  return launched(launch_fmt<rlscan::TdLambda>(f, l, td, stream));
}

rlscan_status impl_gae(rlscan_format f, rlscan_layout l, const void* rewards, const void* values, const uint8_t* terminated,
                       const uint8_t* truncated, const void* bootstrap_value, const void* trunc_bootstrap,
                       void* advantages, void* returns, int64_t E, int64_t T, float gamma, float lambda,
                       hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!rewards || !values || !advantages) return RLSCAN_ERR_NULL;
  if (misaligned(rewards, es) || misaligned(values, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, es * E * T);
  io.add_in(values, es * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T, es)) != RLSCAN_OK)
    return st;
  io.add_out(advantages);
  io.add_out(returns);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(rewards);
  a.v = fp(values);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(bootstrap_value);
  a.tboot = fp(trunc_bootstrap);
  a.out0 = fp(advantages);
  a.out1 = fp(returns);
  a.gamma = gamma;
  a.lam = lambda;
  return launched(launch_fmt<rlscan::Gae>(f, l, a, stream));
}

rlscan_status impl_vtrace(rlscan_format f, rlscan_layout l, const void* rewards, const void* values, const void* log_rhos,
                          const uint8_t* terminated, const uint8_t* truncated, const void* bootstrap_value,
                          const void* trunc_bootstrap, void* vs, void* pg_advantages, int64_t E, int64_t T,
                          float gamma, float lambda, float rho_bar, float c_bar, hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (!finite(rho_bar) || !finite(c_bar) || !(rho_bar > 0.0f) || !(c_bar > 0.0f)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!rewards || !values || !log_rhos || !vs) return RLSCAN_ERR_NULL;
  if (misaligned(rewards, es) || misaligned(values, es) || misaligned(log_rhos, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, es * E * T);
  io.add_in(values, es * E * T);
  io.add_in(log_rhos, es * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T, es)) != RLSCAN_OK)
    return st;
  io.add_out(vs);
  io.add_out(pg_advantages);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(rewards);
  a.v = fp(values);
  a.aux = fp(log_rhos);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(bootstrap_value);
  a.tboot = fp(trunc_bootstrap);
  a.out0 = fp(vs);
  a.out1 = fp(pg_advantages);
  a.gamma = gamma;
  a.lam = lambda;
  a.rho_bar = rho_bar;
  a.c_bar = c_bar;
  return launched(launch_fmt<rlscan::Vtrace>(f, l, a, stream));
}

rlscan_status impl_retrace(rlscan_format f, rlscan_layout l, const void* rewards, const void* q_values, const void* expected_q,
                           const void* pi_prob, const void* mu_prob, const uint8_t* terminated,
                           const uint8_t* truncated, const void* bootstrap_value, const void* trunc_bootstrap,
                           void* q_ret, int64_t E, int64_t T, float gamma, float lambda, hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!rewards || !q_values || !expected_q || !pi_prob || !mu_prob || !q_ret) return RLSCAN_ERR_NULL;
  if (misaligned(rewards, es) || misaligned(q_values, es) || misaligned(expected_q, es) ||
      misaligned(pi_prob, es) || misaligned(mu_prob, es))
    return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, es * E * T);
  io.add_in(q_values, es * E * T);
  io.add_in(expected_q, es * E * T);
  io.add_in(pi_prob, es * E * T);
  io.add_in(mu_prob, es * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T, es)) != RLSCAN_OK)
    return st;
  io.add_out(q_ret);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(rewards);
  a.v = fp(q_values);
  a.aux = fp(expected_q);
  a.pi = fp(pi_prob);
  a.mu = fp(mu_prob);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(bootstrap_value);
  a.tboot = fp(trunc_bootstrap);
  a.out0 = fp(q_ret);
  a.gamma = gamma;
  a.lam = lambda;
  return launched(launch_fmt<rlscan::Retrace>(f, l, a, stream));
}

rlscan_status impl_forward(rlscan_format f, rlscan_layout l, bool traces, const void* x, const uint8_t* terminated,
                           const uint8_t* truncated, const void* init, void* out, int64_t E, int64_t T,
                           float gamma, float lambda, hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!x || !out) return RLSCAN_ERR_NULL;
  if (misaligned(x, es) || misaligned(init, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(x, es * E * T);
  io.add_in(terminated, E * T);
  io.add_in(truncated, E * T);
  io.add_in(init, es * E);
  io.add_out(out);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(x);
  a.term = terminated;
  a.trunc = truncated;
  a.row = fp(init);
  a.out0 = fp(out);
  a.gamma = gamma;
  a.lam = lambda;
  return launched(traces ? launch_fmt<rlscan::EligibilityTrace>(f, l, a, stream)
                         : launch_fmt<rlscan::EpisodicPrefixSum>(f, l, a, stream));
}

// The generic recurrence, optionally cut by a done array (rlscan_linear_scan
// passes none).
rlscan_status impl_linear_scan(rlscan_format f, rlscan_layout l, const void* a_coef, const void* b_coef,
                               const uint8_t* done, const void* carry, void* x, int64_t E, int64_t T, int reverse,
                               hipStream_t stream) {
  const int es = elem_size(f);
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!grid_fits(l, E)) return RLSCAN_ERR_SHAPE;
  if (!a_coef || !b_coef || !x) return RLSCAN_ERR_NULL;
  if (misaligned(a_coef, es) || misaligned(b_coef, es) || misaligned(carry, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(a_coef, es * E * T);
  io.add_in(b_coef, es * E * T);
  io.add_in(done, E * T);
  io.add_in(carry, es * E);
  io.add_out(x);
  if ((st = check_io(io, E, T, es)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = fp(a_coef);
  a.v = fp(b_coef);
  a.term = done;
  a.row = fp(carry);
  a.out0 = fp(x);
  return reverse ? launched(launch_fmt<rlscan::LinearScanReverse>(f, l, a, stream))
                 : launched(launch_fmt<rlscan::LinearScanForward>(f, l, a, stream));
}

// Vector traces over [E,T,D] (or [T,E,D]) features.
rlscan_status impl_traces_vec(rlscan_format f, rlscan_layout l, const void* x, const uint8_t* terminated,
                              const uint8_t* truncated, const void* init, void* traces, int64_t E, int64_t T,
                              int64_t D, float gamma, float lambda, hipStream_t stream) {
  const int es = elem_size(f);
  if (D < 0 || (D > 0 && T >= RLSCAN_MAX_T / D)) return RLSCAN_ERR_SHAPE;  // T*D < 2^30
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if ((st = check_shape(E, T * D)) != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda) || es == 0 || !layout_ok(l)) return RLSCAN_ERR_PARAM;
  if (E * T * D == 0) return RLSCAN_OK;
  if (!rlscan::tv_grid_ok(E, D)) return RLSCAN_ERR_SHAPE;  // one block per row and 64 columns
  if (!x || !traces) return RLSCAN_ERR_NULL;
  if (misaligned(x, es) || misaligned(init, es)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(x, es * E * T * D);
  io.add_in(terminated, E * T);
  io.add_in(truncated, E * T);
  io.add_in(init, es * E * D);
  io.add_out(traces);
  if ((st = check_io(io, E, T * D, es)) != RLSCAN_OK) return st;
  return launched(rlscan::launch_traces_vec((int)f, l == RLSCAN_LAYOUT_TIME_MAJOR, fp(x), terminated, truncated,
                                            fp(init), fp(traces), E, T, D, gamma, lambda, stream));
}

}  // namespace

extern "C" {

const char* rlscan_status_string(rlscan_status s) {
  switch (s) {
    case RLSCAN_OK: return "ok";
    case RLSCAN_ERR_NULL: return "a required pointer is NULL";
    case RLSCAN_ERR_SHAPE: return "invalid shape: E or T negative, T >= 2^30, E*T too large, or a grid past 2^32 - 1 work-items";
    case RLSCAN_ERR_PARAM: return "invalid parameter: non-finite, or outside its range";
    case RLSCAN_ERR_HIP: return "HIP kernel launch failed";
    case RLSCAN_ERR_ALIGN: return "a value pointer is not aligned to its element size";
    case RLSCAN_ERR_ALIAS: return "an output overlaps an input or another output";
  }
  return "unknown status";
}

const char* rlscan_version(void) { return "librlscan 0.1.0 gfx950"; }

rlscan_status rlscan_discounted_returns(const float* rewards, const uint8_t* terminated,
                                        const uint8_t* truncated, const float* bootstrap_value,
                                        const float* trunc_bootstrap, float* returns, int64_t E,
                                        int64_t T, float gamma, hipStream_t stream) {
  return impl_discounted_returns(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, rewards, terminated, truncated, bootstrap_value,
                                 trunc_bootstrap, returns, E, T, gamma, stream);
}

rlscan_status rlscan_td_lambda(const float* rewards, const float* values, const uint8_t* terminated,
                               const uint8_t* truncated, const float* bootstrap_value,
                               const float* trunc_bootstrap, float* returns, int64_t E, int64_t T,
                               float gamma, float lambda, hipStream_t stream) {
  return impl_td_lambda(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, rewards, values, terminated, truncated, bootstrap_value,
                        trunc_bootstrap, returns, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_returns_and_td_lambda(const float* rewards, const float* values,
                                          const uint8_t* terminated, const uint8_t* truncated,
                                          const float* bootstrap_value, const float* trunc_bootstrap,
                                          float* returns, float* td_returns, int64_t E, int64_t T, float gamma,
                                          float lambda, hipStream_t stream) {
  return impl_returns_td_lambda(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, rewards, values, terminated, truncated,
                                bootstrap_value, trunc_bootstrap, returns, td_returns, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_gae(const float* rewards, const float* values, const uint8_t* terminated,
                         const uint8_t* truncated, const float* bootstrap_value,
                         const float* trunc_bootstrap, float* advantages, float* returns, int64_t E,
                         int64_t T, float gamma, float lambda, hipStream_t stream) {
  return impl_gae(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, rewards, values, terminated, truncated, bootstrap_value, trunc_bootstrap,
                  advantages, returns, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_vtrace(const float* rewards, const float* values, const float* log_rhos,
                            const uint8_t* terminated, const uint8_t* truncated,
                            const float* bootstrap_value, const float* trunc_bootstrap, float* vs,
                            float* pg_advantages, int64_t E, int64_t T, float gamma, float lambda,
                            float rho_bar, float c_bar, hipStream_t stream) {
  return impl_vtrace(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, rewards, values, log_rhos, terminated, truncated, bootstrap_value,
                     trunc_bootstrap, vs, pg_advantages, E, T, gamma, lambda, rho_bar, c_bar, stream);
}

rlscan_status rlscan_retrace(const float* rewards, const float* q_values, const float* expected_q,
                             const float* pi_prob, const float* mu_prob, const uint8_t* terminated,
                             const uint8_t* truncated, const float* bootstrap_value,
                             const float* trunc_bootstrap, float* q_ret, int64_t E, int64_t T,
                             float gamma, float lambda, hipStream_t stream) {
  return impl_retrace(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, rewards, q_values, expected_q, pi_prob, mu_prob, terminated, truncated,
                      bootstrap_value, trunc_bootstrap, q_ret, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_eligibility_traces(const float* x, const uint8_t* terminated,
                                        const uint8_t* truncated, const float* init, float* traces,
                                        int64_t E, int64_t T, float gamma, float lambda,
                                        hipStream_t stream) {
  return impl_forward(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, true, x, terminated, truncated, init, traces, E, T, gamma, lambda,
                      stream);
}

rlscan_status rlscan_episodic_prefix_sum(const float* x, const uint8_t* terminated,
                                         const uint8_t* truncated, const float* init, float* sums,
                                         int64_t E, int64_t T, hipStream_t stream) {
  return impl_forward(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, false, x, terminated, truncated, init, sums, E, T, 0.0f, 0.0f, stream);
}

// ---------------------------------------------------------------- storage format and layout
rlscan_status rlscan_discounted_returns_ex(rlscan_format fmt, rlscan_layout layout, const void* rewards,
                                           const uint8_t* terminated, const uint8_t* truncated,
                                           const void* bootstrap_value, const void* trunc_bootstrap, void* returns,
                                           int64_t E, int64_t T, float gamma, hipStream_t stream) {
  return impl_discounted_returns(fmt, layout, rewards, terminated, truncated, bootstrap_value, trunc_bootstrap,
                                 returns, E, T, gamma, stream);
}

rlscan_status rlscan_td_lambda_ex(rlscan_format fmt, rlscan_layout layout, const void* rewards, const void* values,
                                  const uint8_t* terminated, const uint8_t* truncated, const void* bootstrap_value,
                                  const void* trunc_bootstrap, void* returns, int64_t E, int64_t T, float gamma,
                                  float lambda, hipStream_t stream) {
  return impl_td_lambda(fmt, layout, rewards, values, terminated, truncated, bootstrap_value, trunc_bootstrap,
                        returns, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_returns_and_td_lambda_ex(rlscan_format fmt, rlscan_layout layout, const void* rewards,
                                             const void* values, const uint8_t* terminated, const uint8_t* truncated,
                                             const void* bootstrap_value, const void* trunc_bootstrap, void* returns,
                                             void* td_returns, int64_t E, int64_t T, float gamma, float lambda,
                                             hipStream_t stream) {
  return impl_returns_td_lambda(fmt, layout, rewards, values, terminated, truncated, bootstrap_value,
                                trunc_bootstrap, returns, td_returns, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_gae_ex(rlscan_format fmt, rlscan_layout layout, const void* rewards, const void* values,
                            const uint8_t* terminated, const uint8_t* truncated, const void* bootstrap_value,
                            const void* trunc_bootstrap, void* advantages, void* returns, int64_t E, int64_t T,
                            float gamma, float lambda, hipStream_t stream) {
  return impl_gae(fmt, layout, rewards, values, terminated, truncated, bootstrap_value, trunc_bootstrap, advantages,
                  returns, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_vtrace_ex(rlscan_format fmt, rlscan_layout layout, const void* rewards, const void* values,
                               const void* log_rhos, const uint8_t* terminated, const uint8_t* truncated,
                               const void* bootstrap_value, const void* trunc_bootstrap, void* vs, void* pg_advantages,
                               int64_t E, int64_t T, float gamma, float lambda, float rho_bar, float c_bar,
                               hipStream_t stream) {
  return impl_vtrace(fmt, layout, rewards, values, log_rhos, terminated, truncated, bootstrap_value, trunc_bootstrap,
                     vs, pg_advantages, E, T, gamma, lambda, rho_bar, c_bar, stream);
}

rlscan_status rlscan_retrace_ex(rlscan_format fmt, rlscan_layout layout, const void* rewards, const void* q_values,
                                const void* expected_q, const void* pi_prob, const void* mu_prob,
                                const uint8_t* terminated, const uint8_t* truncated, const void* bootstrap_value,
                                const void* trunc_bootstrap, void* q_ret, int64_t E, int64_t T, float gamma,
                                float lambda, hipStream_t stream) {
  return impl_retrace(fmt, layout, rewards, q_values, expected_q, pi_prob, mu_prob, terminated, truncated,
                      bootstrap_value, trunc_bootstrap, q_ret, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_eligibility_traces_ex(rlscan_format fmt, rlscan_layout layout, const void* x,
                                           const uint8_t* terminated, const uint8_t* truncated, const void* init,
                                           void* traces, int64_t E, int64_t T, float gamma, float lambda,
                                           hipStream_t stream) {
  return impl_forward(fmt, layout, true, x, terminated, truncated, init, traces, E, T, gamma, lambda, stream);
}

rlscan_status rlscan_episodic_prefix_sum_ex(rlscan_format fmt, rlscan_layout layout, const void* x,
                                            const uint8_t* terminated, const uint8_t* truncated, const void* init,
                                            void* sums, int64_t E, int64_t T, hipStream_t stream) {
  return impl_forward(fmt, layout, false, x, terminated, truncated, init, sums, E, T, 0.0f, 0.0f, stream);
}

rlscan_status rlscan_linear_scan(const float* a_coef, const float* b_coef, const float* carry, float* x,
                                 int64_t E, int64_t T, int reverse, hipStream_t stream) {
  return impl_linear_scan(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, a_coef, b_coef, nullptr, carry, x, E, T,
                          reverse, stream);
}

rlscan_status rlscan_linear_scan_segmented(const float* a_coef, const float* b_coef, const uint8_t* done,
                                           const float* carry, float* x, int64_t E, int64_t T, int reverse,
                                           hipStream_t stream) {
  return impl_linear_scan(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, a_coef, b_coef, done, carry, x, E, T,
                          reverse, stream);
}

rlscan_status rlscan_linear_scan_segmented_ex(rlscan_format fmt, rlscan_layout layout, const void* a_coef,
                                              const void* b_coef, const uint8_t* done, const void* carry, void* x,
                                              int64_t E, int64_t T, int reverse, hipStream_t stream) {
  return impl_linear_scan(fmt, layout, a_coef, b_coef, done, carry, x, E, T, reverse, stream);
}

rlscan_status rlscan_eligibility_traces_vec(const float* x, const uint8_t* terminated, const uint8_t* truncated,
                                            const float* init, float* traces, int64_t E, int64_t T, int64_t D,
                                            float gamma, float lambda, hipStream_t stream) {
  return impl_traces_vec(RLSCAN_FORMAT_F32, RLSCAN_LAYOUT_ENV_MAJOR, x, terminated, truncated, init, traces, E, T,
                         D, gamma, lambda, stream);
}

rlscan_status rlscan_eligibility_traces_vec_ex(rlscan_format fmt, rlscan_layout layout, const void* x,
                                               const uint8_t* terminated, const uint8_t* truncated, const void* init,
                                               void* traces, int64_t E, int64_t T, int64_t D, float gamma,
                                               float lambda, hipStream_t stream) {
  return impl_traces_vec(fmt, layout, x, terminated, truncated, init, traces, E, T, D, gamma, lambda, stream);
}

}  // extern "C"
