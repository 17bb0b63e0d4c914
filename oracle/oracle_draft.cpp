// DSpark hot path, CPU oracle: semi-autoregressive Markov-head drafting and the
// confidence head.  TEST INFRASTRUCTURE ONLY (see oracle.h).
//
// Blog, "Markov sequential head": the draft law at position k is
// softmax(U_k(v) + B(x_{k-1}, v)) with the low-rank transition B = W1 W2, so the
// bias row of the previous token is W1[x_{k-1}, :] W2.  KB section 2: the block is
// sampled left to right from the anchor x_0, and the block law is the product
// of these normalized conditionals.  Bangkok 4.1: rank 256 by default.
#include <cmath>
#include <vector>

#include "oracle.h"
#include "oracle_internal.h"

std::vector<double> orc_internal_draft_logits(int V, int r, int dt, double temp,
                                              const void *U_row, const void *W1,
                                              const void *W2, int prev) {
  std::vector<double> w1(r);
  for (int i = 0; i < r; ++i) w1[i] = orc_internal_widen(dt, W1, (int64_t)prev * r + i);
  std::vector<double> z(V);
  for (int v = 0; v < V; ++v) {
    // bias B(prev, v) = sum_i W1[prev, i] * W2[i, v]; W2 is stored column-major,
    // so W2[i, v] sits at v * r + i.
    double bias = 0.0;
    for (int i = 0; i < r; ++i) bias += w1[i] * orc_internal_widen(dt, W2, (int64_t)v * r + i);
    z[v] = (orc_internal_widen(dt, U_row, v) + bias) / temp;
  }
  return z;
}

extern "C" int orc_draft_position(int V, int r, int dt, double temp, const void *U_row,
                                  const void *W1, const void *W2, int prev, double u,
                                  double *q, double *cdf, double *m, double *S, double *qx) {
  if (V < 1 || r < 1 || prev < 0 || prev >= V || !(temp > 0.0)) return -1;
  std::vector<double> z = orc_internal_draft_logits(V, r, dt, temp, U_row, W1, W2, prev);
  double mz, Sz;
  orc_internal_stats(z, &mz, &Sz);
  std::vector<double> e(V);
  for (int v = 0; v < V; ++v) e[v] = std::exp(z[v] - mz);
  // inverse CDF on the unnormalized masses: smallest v with u*S < sum_{w<=v} e_w
  int x = orc_inverse_cdf(V, e.data(), u, cdf);
  if (q)
    for (int v = 0; v < V; ++v) q[v] = e[v] / Sz;
  if (m) *m = mz;
  if (S) *S = Sz;
  if (qx) *qx = x >= 0 ? e[x] / Sz : NAN;
  return x;
}

extern "C" double orc_conf_head(int d, int r, int dt, const void *h_row, const float *w, float b,
                                double T, const void *W1, int prev) {
  // linear layer on the concatenation [h_k ; W1[x_{k-1}]], then the
  // position's temperature, then a sigmoid
  double s = (double)b;
  for (int j = 0; j < d; ++j) s += (double)w[j] * orc_internal_widen(dt, h_row, j);
  for (int i = 0; i < r; ++i)
    s += (double)w[d + i] * orc_internal_widen(dt, W1, (int64_t)prev * r + i);
  return 1.0 / (1.0 + std::exp(-s / T));
}

extern "C" int orc_draft_request(int gamma, int V, int r, int dt, double temp, const void *U_req,
                                 const void *W1, const void *W2, int x0, const int32_t *x_cond,
                                 const void *h_req, int d, const float *w_conf, float b_conf,
                                 const float *conf_temp, uint64_t seed, uint64_t round, int rho,
                                 int32_t *x, double *qx,
                                 double *m, double *S, double *c) {
  if (gamma < 1 || x0 < 0 || x0 >= V) return -1;
  int prev = x0;
  for (int k = 1; k <= gamma; ++k) {
    if (k > 1) prev = x_cond ? x_cond[k - 2] : x[k - 2];
    if (prev < 0 || prev >= V) return -1;
    const void *U_row = orc_internal_row(dt, U_req, k - 1, V);
    double u = orc_uniform(seed, round, (uint64_t)k, (uint64_t)rho, ORC_STREAM_DRAFT);
    int xk = orc_draft_position(V, r, dt, temp, U_row, W1, W2, prev, u, nullptr, nullptr,
                                m ? &m[k - 1] : nullptr, S ? &S[k - 1] : nullptr,
                                qx ? &qx[k - 1] : nullptr);
    if (xk < 0) return -1;
    x[k - 1] = xk;
    if (h_req && c) {
      const void *h_row = orc_internal_row(dt, h_req, k - 1, d);
      const double T = conf_temp ? (double)conf_temp[k - 1] : 1.0;
      if (!(T > 0.0) || !std::isfinite(T)) return -1;
      c[k - 1] = orc_conf_head(d, r, dt, h_row, w_conf, b_conf, T, W1, prev);
    }
  }
  return 0;
}
