/*
 * DSpark per-round hot path: plain CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * This library is the correctness reference for the HIP library.  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it; the product path never does.  It shares no source with the HIP
 * library.  Everything is single-threaded and written for reading, not
 * speed: floating point is widened exactly to fp64 and computed in fp64,
 * except where a step's result is an integer decision that the method defines
 * on fp32 values (the survival products, see orc_schedule).
 *
 * Sources (the four web pages on the DSpark paper, arXiv 2607.05147):
 *   [Blog]   numb3r33 blog, "DSpark: confidence-scheduled speculative decoding"
 *   [Bangkok] vllmbangkok blog, "DSpark"
 *   [KB]     edgeai1 speculative-decoding knowledge base, "DSpark 精读"
 *   [Reaper] mkdocs.reaper.mx, "3 · DSpark"
 *
 * Notation: q = draft law, p = target law (Blog, "One-token exactness").
 * R requests (index rho), block length gamma, positions k = 1..gamma,
 * vocabulary V, low-rank factor rank r, temperature T.
 *
 * Element types: ORC_F32 = IEEE binary32, ORC_BF16 = bfloat16 bit patterns
 * stored as uint16 (widened exactly by placing them in the high half of a
 * binary32).
 *
 * Layouts (row-major unless said otherwise):
 *   U   [R][gamma][V]  draft base logits U_k
 *   W1  [V][r]         row x is W1[x,:]
 *   W2  column-major r x V: element (i, v) of W2 at W2[v*r + i]
 *   P   flattened target logits, one row per verified position
 */
#ifndef DSPARK_ORACLE_H
#define DSPARK_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_STREAM_DRAFT = 0, ORC_STREAM_ACCEPT = 1, ORC_STREAM_FINAL = 2 };
enum { ORC_SCHED_OFF = 0, ORC_SCHED_EARLY_STOP = 1, ORC_SCHED_FULL_SEARCH = 2,
       ORC_SCHED_ASYNC_TOPK = 3, ORC_SCHED_THRESHOLD = 4 };

/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11): 10 rounds of the 4x64 Philox S-box with the
 * published multipliers and Weyl key increments. */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);

/* The uniform the method draws at (position, request, stream) of a round:
 * counter = (pos, req, stream, round), key = (seed, 0); u = (out0 >> 40) * 2^-24,
 * a multiple of 2^-24 in [0, 1). */
double orc_uniform(uint64_t seed, uint64_t round, uint64_t pos, uint64_t req, uint64_t stream);

/* Widen n elements of type dt to fp64. */
void orc_widen(int dt, const void *src, int64_t n, double *dst);

/* Softmax statistics of a scaled logit row z = x / T: m = max z, S = sum e^{z-m}.
 * Returns 0, or -1 if V < 1. */
int orc_row_stats(int V, int dt, double temp, const void *row, double *m, double *S);

/* Inverse-CDF draw from non-negative masses w[0..V): the smallest v with
 * u * sum(w) < sum_{v' <= v} w[v'] (prefix summed left to right).  If rounding
 * leaves no crossing, the last v with positive mass.  Returns -1 if the total
 * mass is not positive.  cdf (optional) receives the normalized prefix sums. */
int orc_inverse_cdf(int V, const double *w, double u, double *cdf);

/* Markov head, one position (Blog "Markov sequential head"; KB section 2):
 * z_v = (U_k(v) + sum_i W1[prev, i] W2[i, v]) / T, q_k = softmax(z).
 * Draws x_k by inverse CDF with the given uniform.  Outputs: the law q[V]
 * (optional), its cdf[V] (optional), m and S of z, and q(x_k).  Returns x_k,
 * or -1 on bad arguments. */
int orc_draft_position(int V, int r, int dt, double temp,
                       const void *U_row, const void *W1, const void *W2,
                       int prev, double u,
                       double *q, double *cdf, double *m, double *S, double *qx);

/* Confidence head (Bangkok 4.2.1; KB section 4): z = sum_j w[j] h[j] +
 * sum_i w[d + i] W1[prev, i] + b, linear over the concatenation
 * [h_k ; W1[x_{k-1}]], then c = sigmoid(z / T) with the position's
 * temperature T > 0 (sequential temperature scaling, Blog "Sequential
 * temperature scaling"; Bangkok 4.2.1; T = 1 is the uncalibrated head). */
double orc_conf_head(int d, int r, int dt, const void *h_row, const float *w,
                     float b, double T, const void *W1, int prev);

/* Whole draft of one request with the oracle's own samples.  x0 is the anchor.
 * Outputs x[gamma], qx[gamma], m[gamma], S[gamma] and, if h != NULL,
 * c[gamma] from the confidence head.  If x_cond != NULL, position k conditions on
 * x_cond[k-2] instead of the oracle's own previous sample (stage-by-stage
 * comparison); the draw at k is still the oracle's own. */
int orc_draft_request(int gamma, int V, int r, int dt, double temp,
                      const void *U_req /*[gamma][V]*/, const void *W1, const void *W2,
                      int x0, const int32_t *x_cond,
                      const void *h_req /*[gamma][d] or NULL*/, int d, const float *w_conf,
                      float b_conf, const float *conf_temp /*[gamma] or NULL = 1*/,
                      uint64_t seed, uint64_t round, int rho,
                      int32_t *x, double *qx, double *m, double *S, double *c);

/* Forward-only training reductions (Blog "Training objective"; KB section 5),
 * teacher-forced: position k of request rho conditions on x_{k-1} with x_0 =
 * x0[rho] and x_{k-1} = y[rho][k-2] (y [R][gamma] are the ground-truth tokens).
 * q_k = the draft law of orc_draft_position, p_k = softmax(P_row / T) with P in
 * the verify layout (row rho (gamma + 1) + k - 1; the last row of a request is
 * not read); CE_k = -log q_k(y_k); L1_k = sum_v |p_k(v) - q_k(v)|;
 * BCE_k = -(c*_k log c_k + (1 - c*_k) log(1 - c_k)) with c*_k = sum_v min(p, q);
 * w_k = exp(-(k - 1) / gamma); L_x = (1/R) sum_rho sum_k w_k L_x,k / sum_k w_k;
 * totals = (L_ce, L_tv, L_conf, a_ce L_ce + a_tv L_tv + a_conf L_conf).
 * per_pos (optional) receives [3][R][gamma] (CE, L1, BCE). */
int orc_train_losses(int R, int gamma, int V, int r, int dt, double temp, const void *U,
                     const void *W1, const void *W2, const int32_t *x0, const int32_t *y,
                     const void *P, const float *c, double a_ce, double a_tv, double a_conf,
                     double *per_pos, double *totals);

/* TV overlap label (Blog "Total variation label"): sum_v min(p(v), q(v)) for
 * p = softmax(P_row / T), q = softmax(Q_row / T).  Also returns, through tv
 * (optional), 1/2 ||p - q||_1 computed separately. */
double orc_overlap(int V, int dt, double temp, const void *P_row, const void *Q_row, double *tv);

/* Admission rule on an explicit throughput sequence theta[0..N] (Blog
 * "Scheduler objective"; KB section 4): EARLY_STOP returns the first n with
 * n == N or theta[n+1] <= theta[n]; FULL_SEARCH the smallest n maximizing theta.
 * Returns -1 for another mode. */
int orc_select_n(const double *theta, int N, int mode);

/* Confidence scheduler (Blog "Greedy prefix allocation", "Async scheduler in
 * practice"; Bangkok 4.2.2; KB section 4; Reaper 3.3).
 * a[rho][j] = fl32(a[rho][j-1] * c[rho][j]) with a[rho][0] = 1 (binary32,
 * left to right); candidates (rho, j) sorted by (a desc, j asc, rho asc);
 * A_n = sum of the first n floor(a * 2^32) as int64; tau_n = R + A_n 2^-32;
 * theta_n = tau_n * SPS[R + n]; n* by mode (ASYNC_TOPK: K = FULL_SEARCH n*
 * computed on c_prev2, then the top K of the current order).  Outputs ell[R],
 * row_offset[R+1] (exclusive scan of 1 + ell), a[R][gamma] (optional),
 * n_admitted, theta (theta_{n*}; NaN in OFF mode without c).
 * theta_plain (optional) receives theta_{n*'} of the same rule computed with a
 * plain fp64 running sum of a instead of the fixed-point sum, and n_plain its n*'.
 * THRESHOLD (the static confidence cutoff the pages test before the scheduler,
 * Bangkok 5.3; KB section 7): request rho keeps its leading positions whose
 * confidence c[rho][j] >= threshold, up to the first one below it (the kept
 * tokens stay a prefix); n* = sum ell; theta = tau * SPS[R + n*] with tau over
 * the kept positions, or NaN without SPS (SPS is optional in this mode).
 * Returns 0, or -1 on bad arguments (c outside [0, 1], SPS too short). */
int orc_schedule(int R, int gamma, int mode, double threshold, const float *c, const float *c_prev2,
                 const double *SPS, int B_max, int32_t *ell, int32_t *row_offset,
                 float *a, int32_t *n_admitted, double *theta,
                 int32_t *n_plain, double *theta_plain);

/* Brute force over every ell in [0, gamma]^R (R, gamma small): the maximum of
 * tau(ell) * SPS[R + sum ell] with tau(ell) = R + 2^-32 sum_rho sum_{j <= ell_rho}
 * floor(a[rho][j] 2^32), a as in orc_schedule.  Returns the maximum, and the
 * maximizing ell with the smallest total through ell_best (optional). */
double orc_schedule_bruteforce(int R, int gamma, const float *c, const double *SPS,
                               int B_max, int32_t *ell_best);

/* Exact speculative-sampling verification of one request (Blog "One-token
 * exactness", "Why only the longest accepted prefix survives", "Prefix survival
 * and accepted length"; KB section 8).
 *   P_req  [ell + 1][V] target logits of positions 1..ell+1
 *   U_req  [gamma][V]   draft base logits; q_k is recomputed from x_{k-1}
 *   x      [gamma]      drafted tokens (x_0 = anchor x0)
 * For k <= ell: acc_k = [u_acc(k) q_k(x_k) < p_k(x_k)], c*_k = sum_v min(p_k, q_k).
 * n = (first rejected k) - 1, or ell.  If n < ell the final token is drawn from
 * (p_{n+1} - q_{n+1})_+ (from p_{n+1} if that mass is not positive), else the
 * bonus token from p_{ell+1}; both by inverse CDF with u_final(position).
 * force_n >= 0 replaces n for the final draw (stage-by-stage comparison).
 * Outputs: n_acc, y[gamma + 1] (x_1..x_n, final, then -1), c_star[gamma] (NaN
 * beyond ell), and diagnostics (optional): ratio[gamma] = p_k(x_k)/q_k(x_k),
 * u_acc[gamma], final_cdf[V] = normalized CDF of the final law, final_u,
 * residual_fallback (1 if the residual mass was not positive).
 * Returns 0, or -1 on bad arguments. */
int orc_verify_request(int gamma, int V, int r, int dt, double temp, int ell,
                       const void *P_req, const void *U_req, const void *W1, const void *W2,
                       int x0, const int32_t *x, uint64_t seed, uint64_t round, int rho,
                       int force_n,
                       int32_t *n_acc, int32_t *y, double *c_star,
                       double *ratio, double *u_acc, double *final_cdf, double *final_u,
                       int32_t *residual_fallback);

/* As orc_verify_request, with the draft's transition row of position k taken
 * from row k - 1 of A_rows [gamma][r] (dt) instead of W1[x_{k-1}]. */
int orc_verify_request_rows(int gamma, int V, int r, int dt, double temp, int ell,
                            const void *P_req, const void *U_req, const void *A_rows,
                            const void *W2, int x0, const int32_t *x, uint64_t seed,
                            uint64_t round, int rho, int force_n, int32_t *n_acc, int32_t *y,
                            double *c_star, double *ratio, double *u_acc, double *final_cdf,
                            double *final_u, int32_t *residual_fallback);

/* Recurrent sequential head (Blog "RNN sequential head"; KB section 3): the
 * state s_k = f(s_{k-1}, E(x_{k-1}), h_k) with f a gated recurrent unit, read
 * as the standard GRU (reset gate, update gate, candidate):
 *   g = G_E[x_{k-1}] + G_h[k-1]            input pre-activations [3r]
 *   a = W_hh s_{k-1} + b_hh                 recurrent pre-activations [3r]
 *   rg = sigmoid(g_r + a_r), zg = sigmoid(g_z + a_z)
 *   n  = tanh(g_n + rg * a_n)
 *   s_k = (1 - zg) * n + zg * s_{k-1}
 * G_E [V][3r] (dt) is the input projection of the token embedding table, G_h
 * [gamma][3r] fp32 that of the backbone hidden states (input biases folded
 * in), W_hh column-major [r][3r] (dt, element (g, i) at W_hh[i * 3r + g]),
 * b_hh [3r] fp32, s0 [r] fp32 or NULL (zeros).  Tokens: x_0 = x0, x_k = x[k-1].
 * Output s_out [gamma][r] in fp64.  Returns 0, or -1 on bad arguments. */
int orc_rnn_states(int gamma, int V, int r, int dt, const void *G_E, const float *G_h,
                   const void *W_hh, const float *b_hh, int x0, const int32_t *x,
                   const float *s0, double *s_out);

#ifdef __cplusplus
}
#endif
#endif
