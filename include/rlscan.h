/*
 * rlscan.h -- C ABI of librlscan: RL credit-assignment estimators on MI355X
 * (gfx950) as one-pass affine scans.
 *
 * Every estimator below is the first-order linear recurrence
 *     x_t = a_t * x_{t+1} + b_t            (backward in time)
 * or its forward-time mirror  x_t = a_t * x_{t-1} + b_t, with the per-step
 * coefficients (a_t, b_t) built on-chip from the raw rollout inputs and the
 * recurrence solved by an associative scan over (a, b) pairs.  Source: rl-triton
 * (arxivlens.com paper view), Abstract; gist.science summary of rl-triton,
 * "Technische Samenvatting" > "Methodologie" section 1 (Unified Algebraic
 * Framework: the recurrence and the pair operator) and section 2 (Fused
 * kernels: coefficients built in registers, one HBM read and one HBM write).
 * The pages name the estimators but give no per-estimator formula; each
 * function names the published definition it computes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout      All [E,T] arrays are row-major and contiguous: row e is
 *             environment e, column t is time step t, element (e,t) sits at
 *             index e*T + t.  [E] arrays hold one value per row.
 * Memory      Every array pointer is a DEVICE pointer (memory the GPU can
 *             read/write, e.g. from hipMalloc or a torch CUDA tensor).  float
 *             pointers must be 4-byte aligned.  The caller owns and allocates
 *             every buffer; the library allocates nothing, keeps no state
 *             between calls and is safe to call from several host threads.
 * Types       Values are IEEE float32 (the _ex entries also take bfloat16
 *             or float16 storage and a time-major layout, see below); flags
 *             are uint8 with nonzero = true.  The scan runs in float64 on-chip and each output is
 *             rounded once to float32 (round to nearest).
 * Flags       terminated[e,t] / truncated[e,t] describe transition t (the same
 *             index as reward t).  Terminated: the successor state's value is
 *             0.  Truncated: the successor's value is trunc_bootstrap[e,t].  If
 *             both are set, terminated wins.  At the window end t = T-1 of a
 *             step that is neither, the successor's value is
 *             bootstrap_value[e].  The bootstrap always enters the local term
 *             b_t of the cut step and the scan carry beyond the window is 0,
 *             so nothing is counted twice (gist.science summary, "Methodologie"
 *             section 3, Explicit boundary semantics: termination vs
 *             truncation, rollout windows).
 * Optional    A NULL terminated/truncated array means "no such flags" and is
 *             not read.  A NULL bootstrap_value, trunc_bootstrap, init or carry
 *             means zeros.  Outputs documented as optional may be NULL.
 * Streams     Each call validates its arguments on the host, then enqueues its
 *             kernels on `stream` (NULL = the default stream) and returns; it
 *             never synchronises.  Outputs are valid once the stream has
 *             reached that point.  Most calls are one kernel.  Rows of 16384
 *             steps or more, 64 rows or fewer, are split into segments scanned
 *             in parallel by three kernels in turn; until the last of them, the
 *             first output array holds per-segment intermediate values (so it
 *             must not be read or shared before the stream reaches the end of
 *             the call, which the rule above already implies).
 * Errors      Validation happens before any HIP call and returns:
 *               RLSCAN_ERR_SHAPE  E < 0, T < 0, T >= RLSCAN_MAX_T (2^30),
 *                                 E*T overflows int64, or the launch grid
 *                                 would pass 2^32 - 1 work-items: time-major
 *                                 calls with ceil(E/64) > 4194303 (about
 *                                 2^28 environments), vector traces with
 *                                 E*ceil(D/64) > 16777215;
 *               RLSCAN_ERR_PARAM  a parameter is non-finite or out of range;
 *               RLSCAN_ERR_NULL   a required pointer is NULL while E*T > 0;
 *               RLSCAN_ERR_ALIGN  a value pointer is not aligned to its element
 *                                 size (4 bytes for float32, 2 for the 16-bit
 *                                 storage formats);
 *               RLSCAN_ERR_ALIAS  an output range overlaps an input range or
 *                                 another output range;
 *             E*T == 0 (after shape/parameter checks) is a no-op returning
 *             RLSCAN_OK.  A failed launch returns RLSCAN_ERR_HIP.
 *             Non-finite input values are outside the contract.
 */
#ifndef RLSCAN_H
#define RLSCAN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Longest row (time steps) any entry point accepts: rows are addressed with
 * 32-bit byte offsets. */
#define RLSCAN_MAX_T ((int64_t)1 << 30)

typedef enum rlscan_status {
  RLSCAN_OK = 0,
  RLSCAN_ERR_NULL = 1,
  RLSCAN_ERR_SHAPE = 2,
  RLSCAN_ERR_PARAM = 3,
  RLSCAN_ERR_HIP = 4,
  RLSCAN_ERR_ALIGN = 5,
  RLSCAN_ERR_ALIAS = 6
} rlscan_status;

/* Static, NUL-terminated description of a status code (never NULL). */
const char *rlscan_status_string(rlscan_status status);

/* Static version string, e.g. "librlscan 0.1.0 gfx950". */
const char *rlscan_version(void);

/* Discounted return (Monte-Carlo return with bootstrap at cuts; the
 * discounted return of Sutton & Barto 2018, eq. 3.9, truncated at episode
 * ends and bootstrapped as in section 3 of gist.science's "Methodologie"):
 *   G_t = r_t + gamma * (G_{t+1} while the episode continues, else the
 *         successor value of the cut).
 * Recurrence: a_t = gamma*k_t, b_t = r_t + gamma*(1-k_t)*boot_t, with k_t = 1
 * for a plain continuation and 0 at a cut.
 * In:  rewards [E,T]; terminated, truncated [E,T] (optional);
 *      bootstrap_value [E] (optional); trunc_bootstrap [E,T] (optional, read
 *      only where a step is truncated and not terminated).
 * Out: returns [E,T] (required).
 * gamma in [0,1]. */
rlscan_status rlscan_discounted_returns(const float *rewards, const uint8_t *terminated,
                                        const uint8_t *truncated, const float *bootstrap_value,
                                        const float *trunc_bootstrap, float *returns, int64_t E,
                                        int64_t T, float gamma, hipStream_t stream);

/* TD(lambda) return, recursive lambda-return (Sutton & Barto 2018, ch. 12):
 *   G_t = r_t + gamma * ((1-lambda) V_{t+1} + lambda G_{t+1})  while continuing,
 *   G_t = r_t + gamma * boot_t                                  at a cut.
 * In:  rewards, values [E,T]; flags, bootstraps as for discounted returns.
 * Out: returns [E,T] (required).  gamma, lambda in [0,1]. */
rlscan_status rlscan_td_lambda(const float *rewards, const float *values,
                               const uint8_t *terminated, const uint8_t *truncated,
                               const float *bootstrap_value, const float *trunc_bootstrap,
                               float *returns, int64_t E, int64_t T, float gamma, float lambda,
                               hipStream_t stream);

/* Discounted return and TD(lambda) return of the same rollout in one pass
 * (the two entries above, sharing every input read).  The pages pair these
 * two value targets in their benchmark configurations and name fused kernels
 * that read raw inputs once (gist.science summary of rl-triton,
 * "Methodologie" section 2); reading rewards, flags and bootstraps once for
 * both outputs is that principle applied across two estimators.
 * In:  as rlscan_td_lambda.
 * Out: returns [E,T] (required) = rlscan_discounted_returns;
 *      td_returns [E,T] (required) = rlscan_td_lambda with the same gamma.
 * Rows of whole 256-step tiles (T = 64, 128 or a multiple of 256, arrays
 * 16-byte aligned) take one kernel; other shapes run the two single-output
 * kernels in turn on `stream`.  gamma, lambda in [0,1]. */
rlscan_status rlscan_returns_and_td_lambda(const float *rewards, const float *values,
                                          const uint8_t *terminated, const uint8_t *truncated,
                                          const float *bootstrap_value, const float *trunc_bootstrap,
                                          float *returns, float *td_returns, int64_t E, int64_t T,
                                          float gamma, float lambda, hipStream_t stream);

/* Generalized Advantage Estimation (Schulman et al. 2016):
 *   delta_t = r_t + gamma * nu_t - V_t, nu_t = V_{t+1} while continuing, else
 *             the cut's successor value;
 *   A_t = delta_t + gamma*lambda*A_{t+1} (the A_{t+1} term only while continuing).
 * Out: advantages [E,T] (required); returns [E,T] = A + V (optional, NULL =
 * not written).  gamma, lambda in [0,1]. */
rlscan_status rlscan_gae(const float *rewards, const float *values, const uint8_t *terminated,
                         const uint8_t *truncated, const float *bootstrap_value,
                         const float *trunc_bootstrap, float *advantages, float *returns,
                         int64_t E, int64_t T, float gamma, float lambda, hipStream_t stream);

/* V-trace (Espeholt et al. 2018, IMPALA, eq. 1 with lambda-weighted traces):
 *   ratio_t = exp(log_rhos_t), rho_t = min(rho_bar, ratio_t),
 *   c_t = lambda * min(c_bar, ratio_t),
 *   delta_t = rho_t (r_t + gamma nu_t - V_t),
 *   vs_t - V_t = delta_t + gamma c_t (vs_{t+1} - V_{t+1})  while continuing;
 *   pg_t = rho_t (r_t + gamma * (vs_{t+1} while continuing, else the cut's
 *          successor value) - V_t).
 * In:  rewards, values, log_rhos = log(pi/mu) [E,T]; flags and bootstraps as
 *      above.
 * Out: vs [E,T] (required); pg_advantages [E,T] (optional).
 * gamma, lambda in [0,1] (lambda = 1 is plain IMPALA); rho_bar, c_bar finite
 * and > 0. */
rlscan_status rlscan_vtrace(const float *rewards, const float *values, const float *log_rhos,
                            const uint8_t *terminated, const uint8_t *truncated,
                            const float *bootstrap_value, const float *trunc_bootstrap,
                            float *vs, float *pg_advantages, int64_t E, int64_t T, float gamma,
                            float lambda, float rho_bar, float c_bar, hipStream_t stream);

/* Retrace(lambda) (Munos et al. 2016):
 *   c_{t+1} = lambda * min(1, pi_{t+1} / mu_{t+1}),
 *   Qret_t = r_t + gamma * (EQ_{t+1} + c_{t+1} (Qret_{t+1} - Q_{t+1}))  while continuing,
 *   Qret_t = r_t + gamma * boot_t                                       at a cut.
 * In:  rewards; q_values = Q(s_t, a_t); expected_q = E_pi Q(s_t, .);
 *      pi_prob / mu_prob = target / behaviour probability of a_t (> 0) [E,T];
 *      bootstrap_value [E] = E_pi Q(s_T, .) (optional); flags, trunc_bootstrap
 *      as above.
 * Out: q_ret [E,T] (required).  gamma, lambda in [0,1]. */
rlscan_status rlscan_retrace(const float *rewards, const float *q_values, const float *expected_q,
                             const float *pi_prob, const float *mu_prob, const uint8_t *terminated,
                             const uint8_t *truncated, const float *bootstrap_value,
                             const float *trunc_bootstrap, float *q_ret, int64_t E, int64_t T,
                             float gamma, float lambda, hipStream_t stream);

/* Accumulating eligibility trace, forward in time (the forward-time mirror of
 * the recurrence in the gist.science summary, "Methodologie" section 1):
 *   e_t = gamma*lambda * e_{t-1} + x_t, e_{-1} = init[e] (NULL -> 0), and the
 *   trace restarts from 0 after any step that terminated or was truncated.
 * Out: traces [E,T] (required).  gamma, lambda in [0,1]. */
rlscan_status rlscan_eligibility_traces(const float *x, const uint8_t *terminated,
                                        const uint8_t *truncated, const float *init, float *traces,
                                        int64_t E, int64_t T, float gamma, float lambda,
                                        hipStream_t stream);

/* Eligibility traces of a feature vector per step ([E,T,D] features, e.g. the
 * gradient of the value estimate), forward in time: every column d follows
 * rlscan_eligibility_traces with the row's flags,
 *   e_t[d] = gamma*lambda * (t == 0 ? init[d] : (done_{t-1} ? 0 : e_{t-1}[d])) + x_t[d],
 * done = terminated or truncated (gist.science summary, "Methodologie"
 * section 1 names eligibility traces as the forward-time recurrence; the pages
 * print no vector form, and this entry reads one as the same recurrence run
 * column by column with the row's shared decay and cuts).
 * Layout: x and traces [E,T,D] row-major (element (e,t,d) at (e*T + t)*D + d);
 * terminated, truncated [E,T] (optional); init [E,D] (optional, NULL -> 0).
 * Out: traces [E,T,D] (required).  gamma, lambda in [0,1].  One block of four
 * waves covers 64 columns of a row; full speed needs E*ceil(D/64) blocks in
 * the thousands.
 * Errors as above, with D < 0, T*D >= RLSCAN_MAX_T or E*T*D overflowing
 * reported as RLSCAN_ERR_SHAPE, and so is a grid past 2^32 - 1 work-items
 * (E*ceil(D/64) >= 2^24 blocks), before any HIP call. */
rlscan_status rlscan_eligibility_traces_vec(const float *x, const uint8_t *terminated,
                                            const uint8_t *truncated, const float *init, float *traces,
                                            int64_t E, int64_t T, int64_t D, float gamma, float lambda,
                                            hipStream_t stream);

/* Episodic inclusive prefix sum, forward in time:
 *   S_t = S_{t-1} + x_t, S_{-1} = init[e] (NULL -> 0), restarting from 0 after
 *   any step that terminated or was truncated.
 * Out: sums [E,T] (required). */
rlscan_status rlscan_episodic_prefix_sum(const float *x, const uint8_t *terminated,
                                         const uint8_t *truncated, const float *init, float *sums,
                                         int64_t E, int64_t T, hipStream_t stream);

/* The generic recurrence itself (gist.science summary, "Methodologie"
 * section 1), with caller-supplied coefficients and no flags:
 *   reverse != 0:  x_t = a_t x_{t+1} + b_t,  x_T    = carry[e]
 *   reverse == 0:  x_t = a_t x_{t-1} + b_t,  x_{-1} = carry[e]
 * In:  a, b [E,T] (required); carry [E] (optional, NULL -> 0).
 * Out: x [E,T] (required). */
rlscan_status rlscan_linear_scan(const float *a, const float *b, const float *carry, float *x,
                                 int64_t E, int64_t T, int reverse, hipStream_t stream);

/* The generic recurrence cut into episodes by a flag array: the same
 * recurrence as rlscan_linear_scan, except that a flagged step breaks the
 * chain, as terminated/truncated flags do for the estimators (gist.science
 * summary, "Methodologie" sections 1 and 3):
 *   reverse != 0:  x_t = b_t + (done[t]   ? 0 : a_t x_{t+1}),  x_T    = carry[e]
 *   reverse == 0:  x_t = b_t + (done[t-1] ? 0 : a_t x_{t-1}),  x_{-1} = carry[e]
 * (forward: the step after a flagged one starts a new episode; the carry
 * enters step 0 through a_0 as in rlscan_linear_scan).  done[e,t] is uint8,
 * nonzero = cut; NULL means no cuts (then this equals rlscan_linear_scan).
 * In:  a, b [E,T] (required); done [E,T] (optional); carry [E] (optional).
 * Out: x [E,T] (required). */
rlscan_status rlscan_linear_scan_segmented(const float *a, const float *b, const uint8_t *done,
                                           const float *carry, float *x, int64_t E, int64_t T, int reverse,
                                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Storage format and layout.  The seven estimators, the two-output pass, the
 * vector traces and the generic scan again, each with two more leading
 * arguments; every other argument means what it means for the float32 entry
 * of the same name.
 *
 * fmt     The type of every value array (inputs, bootstraps, init and
 *         outputs): float32, bfloat16 or float16.  16-bit storage halves the
 *         HBM bytes per step; the pages fix no precision, so this is an
 *         extension for rollouts already kept in 16 bits (the gist.science
 *         summary's plain-language part names specialised data formats as
 *         work still to do).  Inputs are widened exactly on load, the scan
 *         runs in float64 as above, and each output is rounded to float32 and
 *         then to the format (round to nearest even both times; float16
 *         overflow gives +-inf).  Flags stay uint8.  Value pointers must be
 *         aligned to the element size (2 bytes for the 16-bit formats).
 * layout  RLSCAN_LAYOUT_ENV_MAJOR: [E,T] arrays as above, (e,t) at e*T + t.
 *         RLSCAN_LAYOUT_TIME_MAJOR: [T,E] arrays, (e,t) at t*E + e, the order
 *         of rollout buffers that append one step for all environments (the
 *         rl-triton skill page, skillsdirectory.com, "Implementation
 *         Workflow" step 2, lists contiguous and strided layouts).  This
 *         applies to rewards, values and every other [E,T] input or output,
 *         flags and trunc_bootstrap included; [E] arrays are unchanged.  E and
 *         T keep their meaning (environments, steps).  Time-major calls run
 *         blocks that each cover 64 environments (one launch; three when
 *         there are fewer groups of 64 than compute units and the columns are
 *         long); full speed needs E in the thousands.  A time-major grid past
 *         2^32 - 1 work-items (ceil(E/64) > 4194303, about 2^28
 *         environments) is refused with RLSCAN_ERR_SHAPE before any HIP
 *         call.
 * An unknown fmt or layout is RLSCAN_ERR_PARAM.  (RLSCAN_FORMAT_F32,
 * RLSCAN_LAYOUT_ENV_MAJOR) is exactly the float32 entry.
 * ------------------------------------------------------------------------ */
typedef enum rlscan_format {
  RLSCAN_FORMAT_F32 = 0,  /* IEEE binary32 */
  RLSCAN_FORMAT_BF16 = 1, /* bfloat16: 8-bit exponent, 7-bit mantissa */
  RLSCAN_FORMAT_F16 = 2   /* IEEE binary16 */
} rlscan_format;

typedef enum rlscan_layout {
  RLSCAN_LAYOUT_ENV_MAJOR = 0, /* [E,T] row-major: (e,t) at e*T + t */
  RLSCAN_LAYOUT_TIME_MAJOR = 1 /* [T,E] row-major: (e,t) at t*E + e */
} rlscan_layout;

rlscan_status rlscan_discounted_returns_ex(rlscan_format fmt, rlscan_layout layout, const void *rewards,
                                           const uint8_t *terminated, const uint8_t *truncated,
                                           const void *bootstrap_value, const void *trunc_bootstrap, void *returns,
                                           int64_t E, int64_t T, float gamma, hipStream_t stream);

rlscan_status rlscan_td_lambda_ex(rlscan_format fmt, rlscan_layout layout, const void *rewards, const void *values,
                                  const uint8_t *terminated, const uint8_t *truncated, const void *bootstrap_value,
                                  const void *trunc_bootstrap, void *returns, int64_t E, int64_t T, float gamma,
                                  float lambda, hipStream_t stream);

/* (16-bit or time-major calls run the two single-output kernels in turn.) */
rlscan_status rlscan_returns_and_td_lambda_ex(rlscan_format fmt, rlscan_layout layout, const void *rewards,
                                             const void *values, const uint8_t *terminated,
                                             const uint8_t *truncated, const void *bootstrap_value,
                                             const void *trunc_bootstrap, void *returns, void *td_returns, int64_t E,
                                             int64_t T, float gamma, float lambda, hipStream_t stream);

rlscan_status rlscan_gae_ex(rlscan_format fmt, rlscan_layout layout, const void *rewards, const void *values,
                            const uint8_t *terminated, const uint8_t *truncated, const void *bootstrap_value,
                            const void *trunc_bootstrap, void *advantages, void *returns, int64_t E, int64_t T,
                            float gamma, float lambda, hipStream_t stream);

rlscan_status rlscan_vtrace_ex(rlscan_format fmt, rlscan_layout layout, const void *rewards, const void *values,
                               const void *log_rhos, const uint8_t *terminated, const uint8_t *truncated,
                               const void *bootstrap_value, const void *trunc_bootstrap, void *vs, void *pg_advantages,
                               int64_t E, int64_t T, float gamma, float lambda, float rho_bar, float c_bar,
                               hipStream_t stream);

rlscan_status rlscan_retrace_ex(rlscan_format fmt, rlscan_layout layout, const void *rewards, const void *q_values,
                                const void *expected_q, const void *pi_prob, const void *mu_prob,
                                const uint8_t *terminated, const uint8_t *truncated, const void *bootstrap_value,
                                const void *trunc_bootstrap, void *q_ret, int64_t E, int64_t T, float gamma,
                                float lambda, hipStream_t stream);

rlscan_status rlscan_eligibility_traces_ex(rlscan_format fmt, rlscan_layout layout, const void *x,
                                           const uint8_t *terminated, const uint8_t *truncated, const void *init,
                                           void *traces, int64_t E, int64_t T, float gamma, float lambda,
                                           hipStream_t stream);

rlscan_status rlscan_episodic_prefix_sum_ex(rlscan_format fmt, rlscan_layout layout, const void *x,
                                            const uint8_t *terminated, const uint8_t *truncated, const void *init,
                                            void *sums, int64_t E, int64_t T, hipStream_t stream);

/* Vector traces (rlscan_eligibility_traces_vec) in a storage format and
 * layout: x, init and traces in format fmt; time-major takes x and traces as
 * [T,E,D] ((e,t,d) at (t*E + e)*D + d) and the flags as [T,E]; init stays
 * [E,D]. */
rlscan_status rlscan_eligibility_traces_vec_ex(rlscan_format fmt, rlscan_layout layout, const void *x,
                                               const uint8_t *terminated, const uint8_t *truncated,
                                               const void *init, void *traces, int64_t E, int64_t T, int64_t D,
                                               float gamma, float lambda, hipStream_t stream);

/* The generic recurrence with episode cuts (rlscan_linear_scan_segmented;
 * done = NULL gives rlscan_linear_scan) in a storage format and layout: a, b,
 * carry and x in format fmt, a, b, done and x in the layout (carry stays
 * [E]). */
rlscan_status rlscan_linear_scan_segmented_ex(rlscan_format fmt, rlscan_layout layout, const void *a, const void *b,
                                              const uint8_t *done, const void *carry, void *x, int64_t E, int64_t T,
                                              int reverse, hipStream_t stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* RLSCAN_H */
