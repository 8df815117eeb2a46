/*
 * rlscan_oracle.c -- fp64 CPU oracle for the RL credit-assignment estimators.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, sequential
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check of the package entry file and the CPU-baseline leg of the
 * benchmark may load it.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code, header or table with it.
 *
 * What is computed (sources):
 *   - The seven estimators named in rl-triton (arxivlens.com paper view),
 *     Abstract, and in the gist.science technical summary of rl-triton,
 *     "Methodologie" section 1 (Unified Algebraic Framework).  Those pages
 *     name the estimators and fix the backward first-order recurrence, but
 *     give no per-estimator formula, so each function below writes out the
 *     standard published recursion, step by step, backward (or forward) in
 *     time:
 *       discounted return  G_t = r_t + gamma * G_{t+1}
 *       TD(lambda) return  Sutton & Barto (2018), recursive lambda-return
 *                          G^l_t = r_t + gamma((1-l)V_{t+1} + l G^l_{t+1})
 *       GAE                Schulman et al. (2016), delta_t and
 *                          A_t = delta_t + gamma*lambda*A_{t+1}
 *       V-trace            Espeholt et al. (2018, IMPALA), eq. (1) with the
 *                          lambda-weighted traces c_i = lambda*min(cbar, pi/mu)
 *                          and the policy-gradient advantage of section 4.2
 *       Retrace(lambda)    Munos et al. (2016), recursive target with traces
 *                          c_s = lambda*min(1, pi/mu)
 *       eligibility trace  accumulating trace e_t = gamma*lambda*e_{t-1} + x_t,
 *                          forward in time (the forward-time mirror named in
 *                          the same gist.science section)
 *       episodic prefix    S_t = S_{t-1} + x_t, forward, reset per episode
 *       generic scan       x_t = a_t x_{t+1} + b_t  (or forward mirror), and
 *                          the same recurrence cut at flagged steps
 *       vector traces      the eligibility trace of every column of an
 *                          [E,T,D] feature array, with the row's flags
 *   - Episode boundaries follow gist.science "Methodologie" section 3
 *     (Expliciete Boundary Semantiek): a terminated step has successor value
 *     zero; a truncated step uses a supplied bootstrap value; the rollout
 *     window end t = T-1 uses the per-row bootstrap.  Readings taken where
 *     the pages are silent:
 *       * flags[t] belong to transition t (same index as r[t]);
 *       * when a step is both terminated and truncated, terminated wins;
 *       * truncation at t = T-1 takes trunc_bootstrap[t], not the row
 *         bootstrap; the row bootstrap is used only at a plain window end;
 *       * NULL flag arrays mean "no flags"; NULL bootstrap arrays mean 0;
 *       * forward estimators reset after any terminated-or-truncated step
 *         and take init[e] as the value before t = 0 (NULL -> 0).
 *
 * Pins (tests that check this file against something other than itself):
 * independent direct sums over every flag pattern of short rows and over
 * random rows (every function); closed forms (constant-reward returns,
 * unit-signal traces, integer prefix sums, degenerate generic scans);
 * reductions between estimators (GAE at lambda 0 and 1, TD(lambda) - V =
 * GAE, TD(1) = discounted return, on-policy V-trace = TD(lambda), Retrace at
 * lambda 0 and on-policy); hand-worked examples; per-column equality of the
 * vector traces with the scalar traces; and planted mistakes that each of
 * these must catch.  No function is left without a pin.  The readings above
 * are pinned only to themselves: the pages do not fix them.
 *
 * Precision: inputs are fp32 and are upcast exactly; parameters arrive as
 * float (as in the GPU ABI) and are upcast exactly; all arithmetic is IEEE
 * double, no fast-math; outputs are double.
 *
 * Layout: every [E,T] array is row-major contiguous (row e is env e,
 * column t is time step t); [E] arrays hold one value per env row.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* Step kinds for the backward estimators. */
enum { STEP_CONT = 0, STEP_TERM = 1, STEP_TRUNC = 2, STEP_END = 3 };

static int step_kind(const uint8_t *term, const uint8_t *trunc, int64_t i,
                     int64_t t, int64_t T) {
  if (term && term[i]) return STEP_TERM;
  if (trunc && trunc[i]) return STEP_TRUNC;
  if (t == T - 1) return STEP_END;
  return STEP_CONT;
}

/* Value of the successor state used at a cut (kind != CONT). */
static double cut_bootstrap(int kind, const float *bootstrap_value,
                            const float *trunc_bootstrap, int64_t e,
                            int64_t i) {
  if (kind == STEP_TERM) return 0.0;
  if (kind == STEP_TRUNC) return trunc_bootstrap ? (double)trunc_bootstrap[i] : 0.0;
  /* STEP_END */
  return bootstrap_value ? (double)bootstrap_value[e] : 0.0;
}

/* Forward estimators: did step i end its episode (terminated or truncated)? */
static int step_done(const uint8_t *term, const uint8_t *trunc, int64_t i) {
  return (term && term[i]) || (trunc && trunc[i]);
}

/* Discounted return: G_t = r_t + gamma * (G_{t+1} if the episode continues
 * inside the window, else the bootstrap of the cut). */
void oracle_discounted_returns(const float *r, const uint8_t *term,
                               const uint8_t *trunc,
                               const float *bootstrap_value,
                               const float *trunc_bootstrap, double *returns,
                               int64_t E, int64_t T, float gamma_f) {
  const double gamma = gamma_f;
  for (int64_t e = 0; e < E; ++e) {
    double G_next = 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
      const int64_t i = e * T + t;
      const int kind = step_kind(term, trunc, i, t, T);
      double succ;
      if (kind == STEP_CONT)
        succ = G_next;
      else
        succ = cut_bootstrap(kind, bootstrap_value, trunc_bootstrap, e, i);
      const double G = (double)r[i] + gamma * succ;
      returns[i] = G;
      G_next = G;
    }
  }
}

/* TD(lambda) return, recursive form of the lambda-return:
 * G_t = r_t + gamma * ((1-lambda) V_{t+1} + lambda G_{t+1}) while the
 * episode continues; at a cut the successor is the bootstrap value. */
void oracle_td_lambda(const float *r, const float *v, const uint8_t *term,
                      const uint8_t *trunc, const float *bootstrap_value,
                      const float *trunc_bootstrap, double *returns, int64_t E,
                      int64_t T, float gamma_f, float lambda_f) {
  const double gamma = gamma_f, lambda = lambda_f;
  for (int64_t e = 0; e < E; ++e) {
    double G_next = 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
      const int64_t i = e * T + t;
      const int kind = step_kind(term, trunc, i, t, T);
      double succ;
      if (kind == STEP_CONT)
        succ = (1.0 - lambda) * (double)v[i + 1] + lambda * G_next;
      else
        succ = cut_bootstrap(kind, bootstrap_value, trunc_bootstrap, e, i);
      const double G = (double)r[i] + gamma * succ;
      returns[i] = G;
      G_next = G;
    }
  }
}

/* GAE: delta_t = r_t + gamma * V_next - V_t with V_next = V_{t+1} while the
 * episode continues and the cut bootstrap otherwise;
 * A_t = delta_t + gamma * lambda * A_{t+1} (the A_{t+1} term only while the
 * episode continues).  returns (optional) = A + V. */
void oracle_gae(const float *r, const float *v, const uint8_t *term,
                const uint8_t *trunc, const float *bootstrap_value,
                const float *trunc_bootstrap, double *advantages,
                double *returns, int64_t E, int64_t T, float gamma_f,
                float lambda_f) {
  const double gamma = gamma_f, lambda = lambda_f;
  for (int64_t e = 0; e < E; ++e) {
    double A_next = 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
      const int64_t i = e * T + t;
      const int kind = step_kind(term, trunc, i, t, T);
      double v_next, carry;
      if (kind == STEP_CONT) {
        v_next = (double)v[i + 1];
        carry = A_next;
      } else {
        v_next = cut_bootstrap(kind, bootstrap_value, trunc_bootstrap, e, i);
        carry = 0.0;
      }
      const double delta = (double)r[i] + gamma * v_next - (double)v[i];
      const double A = delta + gamma * lambda * carry;
      advantages[i] = A;
      if (returns) returns[i] = A + (double)v[i];
      A_next = A;
    }
  }
}

/* V-trace (IMPALA).  With rho_t = min(rho_bar, pi/mu), c_t = lambda *
 * min(c_bar, pi/mu) and pi/mu = exp(log_rhos):
 *   delta_t = rho_t (r_t + gamma V_next - V_t)
 *   vs_t - V_t = delta_t + gamma c_t (vs_{t+1} - V_{t+1})   (while continuing)
 *   pg_t = rho_t (r_t + gamma vs_next - V_t), vs_next = vs_{t+1} while
 *          continuing, the cut bootstrap otherwise.
 * The policy-gradient clip uses rho_bar. */
void oracle_vtrace(const float *r, const float *v, const float *log_rhos,
                   const uint8_t *term, const uint8_t *trunc,
                   const float *bootstrap_value, const float *trunc_bootstrap,
                   double *vs, double *pg_advantages, int64_t E, int64_t T,
                   float gamma_f, float lambda_f, float rho_bar_f,
                   float c_bar_f) {
  const double gamma = gamma_f, lambda = lambda_f;
  const double rho_bar = rho_bar_f, c_bar = c_bar_f;
  for (int64_t e = 0; e < E; ++e) {
    double vs_next = 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
      const int64_t i = e * T + t;
      const int kind = step_kind(term, trunc, i, t, T);
      const double ratio = exp((double)log_rhos[i]);
      const double rho = fmin(rho_bar, ratio);
      const double c = lambda * fmin(c_bar, ratio);
      double v_next, diff_next, vs_succ;
      if (kind == STEP_CONT) {
        v_next = (double)v[i + 1];
        diff_next = vs_next - (double)v[i + 1];
        vs_succ = vs_next;
      } else {
        v_next = cut_bootstrap(kind, bootstrap_value, trunc_bootstrap, e, i);
        diff_next = 0.0;
        vs_succ = v_next;
      }
      const double delta = rho * ((double)r[i] + gamma * v_next - (double)v[i]);
      const double vs_t = (double)v[i] + delta + gamma * c * diff_next;
      vs[i] = vs_t;
      if (pg_advantages)
        pg_advantages[i] = rho * ((double)r[i] + gamma * vs_succ - (double)v[i]);
      vs_next = vs_t;
    }
  }
}

/* Retrace(lambda):
 *   Qret_t = r_t + gamma * (E_pi Q(s_{t+1},.) + c_{t+1} (Qret_{t+1} - Q_{t+1}))
 * while the episode continues inside the window, with
 * c_{t+1} = lambda * min(1, pi_{t+1} / mu_{t+1}); at a cut
 *   Qret_t = r_t + gamma * bootstrap.
 * exp_q[t] holds E_pi Q(s_t,.); bootstrap_value[e] holds E_pi Q(s_T,.);
 * pi_prob / mu_prob are the target / behaviour probabilities of the taken
 * action a_t. */
void oracle_retrace(const float *r, const float *q, const float *exp_q,
                    const float *pi_prob, const float *mu_prob,
                    const uint8_t *term, const uint8_t *trunc,
                    const float *bootstrap_value, const float *trunc_bootstrap,
                    double *q_ret, int64_t E, int64_t T, float gamma_f,
                    float lambda_f) {
  const double gamma = gamma_f, lambda = lambda_f;
  for (int64_t e = 0; e < E; ++e) {
    double qret_next = 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
      const int64_t i = e * T + t;
      const int kind = step_kind(term, trunc, i, t, T);
      double target;
      if (kind == STEP_CONT) {
        const double ratio = (double)pi_prob[i + 1] / (double)mu_prob[i + 1];
        const double c_next = lambda * fmin(1.0, ratio);
        target = (double)exp_q[i + 1] + c_next * (qret_next - (double)q[i + 1]);
      } else {
        target = cut_bootstrap(kind, bootstrap_value, trunc_bootstrap, e, i);
      }
      const double qret = (double)r[i] + gamma * target;
      q_ret[i] = qret;
      qret_next = qret;
    }
  }
}

/* Accumulating eligibility trace of the signal x, forward in time:
 *   e_t = gamma*lambda * e_{t-1} + x_t, with e_{-1} = init[e] and the trace
 * reset to 0 after a step that terminated or was truncated. */
void oracle_eligibility_traces(const float *x, const uint8_t *term,
                               const uint8_t *trunc, const float *init,
                               double *traces, int64_t E, int64_t T,
                               float gamma_f, float lambda_f) {
  const double decay = (double)gamma_f * (double)lambda_f;
  for (int64_t e = 0; e < E; ++e) {
    double prev = init ? (double)init[e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const int64_t i = e * T + t;
      if (t > 0 && step_done(term, trunc, i - 1)) prev = 0.0;
      const double cur = decay * prev + (double)x[i];
      traces[i] = cur;
      prev = cur;
    }
  }
}

/* Episodic inclusive prefix sum, forward in time:
 *   S_t = S_{t-1} + x_t, with S_{-1} = init[e] and the sum reset to 0 after
 * a step that terminated or was truncated. */
void oracle_episodic_prefix_sum(const float *x, const uint8_t *term,
                                const uint8_t *trunc, const float *init,
                                double *sums, int64_t E, int64_t T) {
  for (int64_t e = 0; e < E; ++e) {
    double prev = init ? (double)init[e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const int64_t i = e * T + t;
      if (t > 0 && step_done(term, trunc, i - 1)) prev = 0.0;
      const double cur = prev + (double)x[i];
      sums[i] = cur;
      prev = cur;
    }
  }
}

/* Generic first-order linear recurrence (the unified form of the gist.science
 * summary, Methodologie section 1):
 *   reverse != 0:  x_t = a_t x_{t+1} + b_t,  x_T    = carry[e]
 *   reverse == 0:  x_t = a_t x_{t-1} + b_t,  x_{-1} = carry[e]
 * carry NULL -> 0. */
void oracle_linear_scan(const float *a, const float *b, const float *carry,
                        double *x, int64_t E, int64_t T, int reverse) {
  for (int64_t e = 0; e < E; ++e) {
    double state = carry ? (double)carry[e] : 0.0;
    for (int64_t k = 0; k < T; ++k) {
      const int64_t t = reverse ? (T - 1 - k) : k;
      const int64_t i = e * T + t;
      state = (double)a[i] * state + (double)b[i];
      x[i] = state;
    }
  }
}

/* The generic recurrence cut into episodes by a flag array: a flagged step
 * breaks the chain, as the estimators' terminated / truncated flags do
 * (gist.science summary, "Methodologie" sections 1 and 3).
 *   reverse: x_t = b_t + (done[t] ? 0 : a_t x_{t+1}),              x_T    = carry
 *   forward: x_t = b_t + (t > 0 && done[t-1] ? 0 : a_t x_{t-1}),   x_{-1} = carry
 * done == NULL means no cuts. */
void oracle_linear_scan_segmented(const float *a, const float *b, const uint8_t *done,
                                  const float *carry, double *x, int64_t E, int64_t T,
                                  int reverse) {
  for (int64_t e = 0; e < E; ++e) {
    double state = carry ? (double)carry[e] : 0.0;
    for (int64_t k = 0; k < T; ++k) {
      const int64_t t = reverse ? (T - 1 - k) : k;
      const int64_t i = e * T + t;
      int cut = 0;
      if (done) cut = reverse ? (done[i] != 0) : (t > 0 && done[i - 1] != 0);
      state = (cut ? 0.0 : (double)a[i] * state) + (double)b[i];
      x[i] = state;
    }
  }
}

/* Eligibility traces of a feature vector per step: x, out [E,T,D] row-major
 * ((e,t,d) at (e*T + t)*D + d), flags [E,T], init [E,D].  Each column d
 * follows the scalar trace recurrence with the row's flags:
 *   e_t[d] = decay * (t == 0 ? init[d] : (done_{t-1} ? 0 : e_{t-1}[d])) + x_t[d]. */
void oracle_eligibility_traces_vec(const float *x, const uint8_t *term, const uint8_t *trunc,
                                   const float *init, double *out, int64_t E, int64_t T, int64_t D,
                                   float gamma_f, float lambda_f) {
  const double decay = (double)gamma_f * (double)lambda_f;
  for (int64_t e = 0; e < E; ++e) {
    for (int64_t d = 0; d < D; ++d) {
      double prev = init ? (double)init[e * D + d] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        if (t > 0 && step_done(term, trunc, e * T + t - 1)) prev = 0.0;
        const int64_t i = (e * T + t) * D + d;
        const double cur = decay * prev + (double)x[i];
        out[i] = cur;
        prev = cur;
      }
    }
  }
}
