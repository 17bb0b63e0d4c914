// DSpark hot path, CPU oracle: exact speculative-sampling verification of one
// request's drafted block.  TEST INFRASTRUCTURE ONLY (see oracle.h).
//
// Blog, "One-token exactness": a draft x ~ q is accepted with probability
// min(1, p(x)/q(x)); at the first rejection the replacement is drawn from the
// residual r(x) proportional to (p(x) - q(x))_+, never from p itself.
// Blog, "Why only the longest accepted prefix survives": only the accepted
// prefix is kept.  Blog, "Prefix survival and accepted length" and KB section
// 6: when every verified draft is accepted the target adds a bonus token.
// Blog, "Total variation label": c*_k = sum_v min(p_k, q_k) = 1 - TV.
#include <cmath>
#include <vector>

#include "oracle.h"
#include "oracle_internal.h"

// A_rows (or NULL): the draft's transition row of position k is row k - 1 of
// A_rows [gamma][r] instead of W1[x_{k-1}] (a head whose bias row is not a
// table lookup, e.g. the recurrent head's state).
static int verify_impl(int gamma, int V, int r, int dt, double temp, int ell,
                       const void *P_req, const void *U_req, const void *W1, const void *A_rows,
                       const void *W2, int x0, const int32_t *x, uint64_t seed, uint64_t round,
                       int rho, int force_n, int32_t *n_acc, int32_t *y, double *c_star,
                       double *ratio, double *u_acc, double *final_cdf, double *final_u,
                       int32_t *residual_fallback) {
  if (gamma < 1 || V < 1 || ell < 0 || ell > gamma || !(temp > 0.0)) return -1;
  if (x0 < 0 || x0 >= V) return -1;
  for (int k = 0; k < ell; ++k)
    if (x[k] < 0 || x[k] >= V) return -1;

  // Target law of every verified position 1..ell+1, draft law of 1..ell.
  std::vector<std::vector<double>> p(ell + 1), q(ell);
  for (int k = 1; k <= ell + 1; ++k)
    p[k - 1] = orc_internal_softmax(
        orc_internal_scaled_row(V, dt, temp, orc_internal_row(dt, P_req, k - 1, V)));
  for (int k = 1; k <= ell; ++k) {
    const int prev = k == 1 ? x0 : x[k - 2];
    q[k - 1] = orc_internal_softmax(orc_internal_draft_logits(
        V, r, dt, temp, orc_internal_row(dt, U_req, k - 1, V), A_rows ? A_rows : W1, W2,
        A_rows ? k - 1 : prev));
  }

  // Soft confidence target and the accept/reject decisions.
  int n = ell;
  for (int k = 1; k <= gamma; ++k) {
    if (c_star) c_star[k - 1] = NAN;
    if (ratio) ratio[k - 1] = NAN;
    if (u_acc) u_acc[k - 1] = NAN;
  }
  for (int k = 1; k <= ell; ++k) {
    double overlap = 0.0;
    for (int v = 0; v < V; ++v) overlap += std::fmin(p[k - 1][v], q[k - 1][v]);
    if (c_star) c_star[k - 1] = overlap;
    const int xk = x[k - 1];
    const double pk = p[k - 1][xk], qk = q[k - 1][xk];
    const double u = orc_uniform(seed, round, (uint64_t)k, (uint64_t)rho, ORC_STREAM_ACCEPT);
    if (ratio) ratio[k - 1] = pk / qk;
    if (u_acc) u_acc[k - 1] = u;
    // accept with probability min(1, p/q): u * q < p for u uniform on [0, 1)
    const bool accepted = u * qk < pk;
    if (!accepted && n == ell) n = k - 1;  // first rejection
  }
  if (force_n >= 0 && force_n <= ell) n = force_n;

  // Final token: residual at the first rejection, bonus after full acceptance.
  std::vector<double> w(V);
  int fallback = 0;
  const int j = n + 1;  // position of the final token
  if (n < ell) {
    double mass = 0.0;
    for (int v = 0; v < V; ++v) {
      w[v] = std::fmax(p[j - 1][v] - q[j - 1][v], 0.0);
      mass += w[v];
    }
    if (!(mass > 0.0)) {  // only by rounding: a rejection implies p(x) < q(x)
      w = p[j - 1];
      fallback = 1;
    }
  } else {
    w = p[ell];
  }
  const double uf = orc_uniform(seed, round, (uint64_t)j, (uint64_t)rho, ORC_STREAM_FINAL);
  const int final_token = orc_inverse_cdf(V, w.data(), uf, final_cdf);
  if (final_u) *final_u = uf;
  if (residual_fallback) *residual_fallback = fallback;

  *n_acc = n;
  for (int i = 0; i <= gamma; ++i) y[i] = -1;
  for (int i = 0; i < n; ++i) y[i] = x[i];
  y[n] = final_token;
  return final_token >= 0 ? 0 : -1;
}

extern "C" int orc_verify_request(int gamma, int V, int r, int dt, double temp, int ell,
                                  const void *P_req, const void *U_req, const void *W1,
                                  const void *W2, int x0, const int32_t *x, uint64_t seed,
                                  uint64_t round, int rho, int force_n, int32_t *n_acc,
                                  int32_t *y, double *c_star, double *ratio, double *u_acc,
                                  double *final_cdf, double *final_u,
                                  int32_t *residual_fallback) {
  return verify_impl(gamma, V, r, dt, temp, ell, P_req, U_req, W1, nullptr, W2, x0, x, seed,
                     round, rho, force_n, n_acc, y, c_star, ratio, u_acc, final_cdf, final_u,
                     residual_fallback);
}

extern "C" int orc_verify_request_rows(int gamma, int V, int r, int dt, double temp, int ell,
                                       const void *P_req, const void *U_req, const void *A_rows,
                                       const void *W2, int x0, const int32_t *x, uint64_t seed,
                                       uint64_t round, int rho, int force_n, int32_t *n_acc,
                                       int32_t *y, double *c_star, double *ratio, double *u_acc,
                                       double *final_cdf, double *final_u,
                                       int32_t *residual_fallback) {
  if (!A_rows) return -1;
  return verify_impl(gamma, V, r, dt, temp, ell, P_req, U_req, nullptr, A_rows, W2, x0, x, seed,
                     round, rho, force_n, n_acc, y, c_star, ratio, u_acc, final_cdf, final_u,
                     residual_fallback);
}
