// rlscan_api.hip -- the C ABI of librlscan (declared in include/rlscan.h).
//
// Every entry point validates its arguments on the host before touching HIP,
// fills the kernel argument block and enqueues exactly one kernel on the
// caller's stream.  Nothing is allocated and no state is kept.
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

bool misaligned(const float* p) { return p && ((uintptr_t)p % alignof(float)) != 0; }

// Inputs and outputs of one call, for the NULL / alignment / overlap checks.
struct Io {
  const void* in[12];
  int64_t in_bytes[12];
  int n_in = 0;
  float* out[2];
  int n_out = 0;
  void add_in(const void* p, int64_t bytes) {
    if (p) {
      in[n_in] = p;
      in_bytes[n_in] = bytes;
      ++n_in;
    }
  }
  void add_out(float* p) {
    if (p) out[n_out++] = p;
  }
};

rlscan_status check_io(const Io& io, int64_t E, int64_t T) {
  const int64_t fbytes = 4 * E * T;
  for (int i = 0; i < io.n_out; ++i) {
    if (misaligned(io.out[i])) return RLSCAN_ERR_ALIGN;
    const Range ro = span(io.out[i], fbytes);
    for (int j = 0; j < io.n_in; ++j)
      if (overlap(ro, span(io.in[j], io.in_bytes[j]))) return RLSCAN_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(ro, span(io.out[j], fbytes))) return RLSCAN_ERR_ALIAS;
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
rlscan_status common_backward(Io& io, const uint8_t* term, const uint8_t* trunc, const float* boot,
                              const float* tboot, int64_t E, int64_t T) {
  if (misaligned(boot) || misaligned(tboot)) return RLSCAN_ERR_ALIGN;
  io.add_in(term, E * T);
  io.add_in(trunc, E * T);
  io.add_in(boot, 4 * E);
  io.add_in(tboot, 4 * E * T);
  return RLSCAN_OK;
}

}  // namespace

extern "C" {

const char* rlscan_status_string(rlscan_status s) {
  switch (s) {
    case RLSCAN_OK: return "ok";
    case RLSCAN_ERR_NULL: return "a required pointer is NULL";
    case RLSCAN_ERR_SHAPE: return "invalid shape: E or T negative, T >= 2^30, or E*T too large";
    case RLSCAN_ERR_PARAM: return "invalid parameter: non-finite, or outside its range";
    case RLSCAN_ERR_HIP: return "HIP kernel launch failed";
    case RLSCAN_ERR_ALIGN: return "a float pointer is not 4-byte aligned";
    case RLSCAN_ERR_ALIAS: return "an output overlaps an input or another output";
  }
  return "unknown status";
}

const char* rlscan_version(void) { return "librlscan 0.1.0 gfx950"; }

rlscan_status rlscan_discounted_returns(const float* rewards, const uint8_t* terminated,
                                        const uint8_t* truncated, const float* bootstrap_value,
                                        const float* trunc_bootstrap, float* returns, int64_t E,
                                        int64_t T, float gamma, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!rewards || !returns) return RLSCAN_ERR_NULL;
  if (misaligned(rewards)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, 4 * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T)) != RLSCAN_OK)
    return st;
  io.add_out(returns);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = rewards;
  a.term = terminated;
  a.trunc = truncated;
  a.row = bootstrap_value;
  a.tboot = trunc_bootstrap;
  a.out0 = returns;
  a.gamma = gamma;
  return launched(rlscan::launch<rlscan::DiscountedReturn>(a, stream));
}

rlscan_status rlscan_td_lambda(const float* rewards, const float* values, const uint8_t* terminated,
                               const uint8_t* truncated, const float* bootstrap_value,
                               const float* trunc_bootstrap, float* returns, int64_t E, int64_t T,
                               float gamma, float lambda, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!rewards || !values || !returns) return RLSCAN_ERR_NULL;
  if (misaligned(rewards) || misaligned(values)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, 4 * E * T);
  io.add_in(values, 4 * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T)) != RLSCAN_OK)
    return st;
  io.add_out(returns);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = rewards;
  a.v = values;
  a.term = terminated;
  a.trunc = truncated;
  a.row = bootstrap_value;
  a.tboot = trunc_bootstrap;
  a.out0 = returns;
  a.gamma = gamma;
  a.lam = lambda;
  return launched(rlscan::launch<rlscan::TdLambda>(a, stream));
}

rlscan_status rlscan_returns_and_td_lambda(const float* rewards, const float* values,
                                          const uint8_t* terminated, const uint8_t* truncated,
                                          const float* bootstrap_value, const float* trunc_bootstrap,
                                          float* returns, float* td_returns, int64_t E, int64_t T, float gamma,
                                          float lambda, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!rewards || !values || !returns || !td_returns) return RLSCAN_ERR_NULL;
  if (misaligned(rewards) || misaligned(values)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, 4 * E * T);
  io.add_in(values, 4 * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T)) != RLSCAN_OK)
    return st;
  io.add_out(returns);
  io.add_out(td_returns);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = rewards;
  a.v = values;
  a.term = terminated;
  a.trunc = truncated;
  a.row = bootstrap_value;
  a.tboot = trunc_bootstrap;
  a.out0 = returns;
  a.out1 = td_returns;
  a.gamma = gamma;
  a.lam = lambda;
  return launched(rlscan::launch_returns_td_lambda(a, stream));
}

rlscan_status rlscan_gae(const float* rewards, const float* values, const uint8_t* terminated,
                         const uint8_t* truncated, const float* bootstrap_value,
                         const float* trunc_bootstrap, float* advantages, float* returns, int64_t E,
                         int64_t T, float gamma, float lambda, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!rewards || !values || !advantages) return RLSCAN_ERR_NULL;
  if (misaligned(rewards) || misaligned(values)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, 4 * E * T);
  io.add_in(values, 4 * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T)) != RLSCAN_OK)
    return st;
  io.add_out(advantages);
  io.add_out(returns);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = rewards;
  a.v = values;
  a.term = terminated;
  a.trunc = truncated;
  a.row = bootstrap_value;
  a.tboot = trunc_bootstrap;
  a.out0 = advantages;
  a.out1 = returns;
  a.gamma = gamma;
  a.lam = lambda;
  return launched(rlscan::launch<rlscan::Gae>(a, stream));
}

rlscan_status rlscan_vtrace(const float* rewards, const float* values, const float* log_rhos,
                            const uint8_t* terminated, const uint8_t* truncated,
                            const float* bootstrap_value, const float* trunc_bootstrap, float* vs,
                            float* pg_advantages, int64_t E, int64_t T, float gamma, float lambda,
                            float rho_bar, float c_bar, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (!finite(rho_bar) || !finite(c_bar) || !(rho_bar > 0.0f) || !(c_bar > 0.0f)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!rewards || !values || !log_rhos || !vs) return RLSCAN_ERR_NULL;
  if (misaligned(rewards) || misaligned(values) || misaligned(log_rhos)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, 4 * E * T);
  io.add_in(values, 4 * E * T);
  io.add_in(log_rhos, 4 * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T)) != RLSCAN_OK)
    return st;
  io.add_out(vs);
  io.add_out(pg_advantages);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = rewards;
  a.v = values;
  a.aux = log_rhos;
  a.term = terminated;
  a.trunc = truncated;
  a.row = bootstrap_value;
  a.tboot = trunc_bootstrap;
  a.out0 = vs;
  a.out1 = pg_advantages;
  a.gamma = gamma;
  a.lam = lambda;
  a.rho_bar = rho_bar;
  a.c_bar = c_bar;
  return launched(rlscan::launch<rlscan::Vtrace>(a, stream));
}

rlscan_status rlscan_retrace(const float* rewards, const float* q_values, const float* expected_q,
                             const float* pi_prob, const float* mu_prob, const uint8_t* terminated,
                             const uint8_t* truncated, const float* bootstrap_value,
                             const float* trunc_bootstrap, float* q_ret, int64_t E, int64_t T,
                             float gamma, float lambda, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!rewards || !q_values || !expected_q || !pi_prob || !mu_prob || !q_ret) return RLSCAN_ERR_NULL;
  if (misaligned(rewards) || misaligned(q_values) || misaligned(expected_q) || misaligned(pi_prob) ||
      misaligned(mu_prob))
    return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(rewards, 4 * E * T);
  io.add_in(q_values, 4 * E * T);
  io.add_in(expected_q, 4 * E * T);
  io.add_in(pi_prob, 4 * E * T);
  io.add_in(mu_prob, 4 * E * T);
  if ((st = common_backward(io, terminated, truncated, bootstrap_value, trunc_bootstrap, E, T)) != RLSCAN_OK)
    return st;
  io.add_out(q_ret);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = rewards;
  a.v = q_values;
  a.aux = expected_q;
  a.pi = pi_prob;
  a.mu = mu_prob;
  a.term = terminated;
  a.trunc = truncated;
  a.row = bootstrap_value;
  a.tboot = trunc_bootstrap;
  a.out0 = q_ret;
  a.gamma = gamma;
  a.lam = lambda;
  return launched(rlscan::launch<rlscan::Retrace>(a, stream));
}

rlscan_status rlscan_eligibility_traces(const float* x, const uint8_t* terminated,
                                        const uint8_t* truncated, const float* init, float* traces,
                                        int64_t E, int64_t T, float gamma, float lambda,
                                        hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (E * T == 0) return RLSCAN_OK;
  if (!x || !traces) return RLSCAN_ERR_NULL;
  if (misaligned(x) || misaligned(init)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(x, 4 * E * T);
  io.add_in(terminated, E * T);
  io.add_in(truncated, E * T);
  io.add_in(init, 4 * E);
  io.add_out(traces);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = x;
  a.term = terminated;
  a.trunc = truncated;
  a.row = init;
  a.out0 = traces;
  a.gamma = gamma;
  a.lam = lambda;
  return launched(rlscan::launch<rlscan::EligibilityTrace>(a, stream));
}

rlscan_status rlscan_episodic_prefix_sum(const float* x, const uint8_t* terminated,
                                         const uint8_t* truncated, const float* init, float* sums,
                                         int64_t E, int64_t T, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (E * T == 0) return RLSCAN_OK;
  if (!x || !sums) return RLSCAN_ERR_NULL;
  if (misaligned(x) || misaligned(init)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(x, 4 * E * T);
  io.add_in(terminated, E * T);
  io.add_in(truncated, E * T);
  io.add_in(init, 4 * E);
  io.add_out(sums);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = x;
  a.term = terminated;
  a.trunc = truncated;
  a.row = init;
  a.out0 = sums;
  return launched(rlscan::launch<rlscan::EpisodicPrefixSum>(a, stream));
}

rlscan_status rlscan_linear_scan(const float* a_coef, const float* b_coef, const float* carry, float* x,
                                 int64_t E, int64_t T, int reverse, hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (E * T == 0) return RLSCAN_OK;
  if (!a_coef || !b_coef || !x) return RLSCAN_ERR_NULL;
  if (misaligned(a_coef) || misaligned(b_coef) || misaligned(carry)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(a_coef, 4 * E * T);
  io.add_in(b_coef, 4 * E * T);
  io.add_in(carry, 4 * E);
  io.add_out(x);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = a_coef;
  a.v = b_coef;
  a.row = carry;
  a.out0 = x;
  return reverse ? launched(rlscan::launch<rlscan::LinearScanReverse>(a, stream))
                 : launched(rlscan::launch<rlscan::LinearScanForward>(a, stream));
}

rlscan_status rlscan_linear_scan_segmented(const float* a_coef, const float* b_coef, const uint8_t* done,
                                           const float* carry, float* x, int64_t E, int64_t T, int reverse,
                                           hipStream_t stream) {
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if (E * T == 0) return RLSCAN_OK;
  if (!a_coef || !b_coef || !x) return RLSCAN_ERR_NULL;
  if (misaligned(a_coef) || misaligned(b_coef) || misaligned(carry)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(a_coef, 4 * E * T);
  io.add_in(b_coef, 4 * E * T);
  io.add_in(done, E * T);
  io.add_in(carry, 4 * E);
  io.add_out(x);
  if ((st = check_io(io, E, T)) != RLSCAN_OK) return st;
  KernelArgs a = blank(E, T);
  a.r = a_coef;
  a.v = b_coef;
  a.term = done;
  a.row = carry;
  a.out0 = x;
  return reverse ? launched(rlscan::launch<rlscan::LinearScanReverse>(a, stream))
                 : launched(rlscan::launch<rlscan::LinearScanForward>(a, stream));
}

rlscan_status rlscan_eligibility_traces_vec(const float* x, const uint8_t* terminated, const uint8_t* truncated,
                                            const float* init, float* traces, int64_t E, int64_t T, int64_t D,
                                            float gamma, float lambda, hipStream_t stream) {
  if (D < 0 || (D > 0 && T >= RLSCAN_MAX_T / D)) return RLSCAN_ERR_SHAPE;  // T*D < 2^30
  rlscan_status st = check_shape(E, T);
  if (st != RLSCAN_OK) return st;
  if ((st = check_shape(E, T * D)) != RLSCAN_OK) return st;
  if (!in_unit(gamma) || !in_unit(lambda)) return RLSCAN_ERR_PARAM;
  if (E * T * D == 0) return RLSCAN_OK;
  if (!x || !traces) return RLSCAN_ERR_NULL;
  if (misaligned(x) || misaligned(init)) return RLSCAN_ERR_ALIGN;
  Io io;
  io.add_in(x, 4 * E * T * D);
  io.add_in(terminated, E * T);
  io.add_in(truncated, E * T);
  io.add_in(init, 4 * E * D);
  io.add_out(traces);
  if ((st = check_io(io, E, T * D)) != RLSCAN_OK) return st;
  return launched(rlscan::launch_traces_vec(x, terminated, truncated, init, traces, E, T, D, gamma, lambda,
                                            stream));
}

}  // extern "C"
