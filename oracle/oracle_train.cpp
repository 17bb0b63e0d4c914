// DSpark hot path, CPU oracle: forward-only training reductions.  TEST
// INFRASTRUCTURE ONLY (see oracle.h).
//
// Blog, "Training objective": the drafter is trained on three weighted
// losses, L = a_ce L_ce + a_tv L_tv + a_conf L_conf (defaults 0.1, 0.9, 1.0),
// with position weights w_k = exp(-(k - 1) / gamma) that favour early
// positions.  KB section 5: hard cross-entropy, an L1 distance between the
// target and draft distributions (twice the total variation, which is what
// sets the acceptance rate) and a binary cross-entropy of the confidence
// against the soft label c*.  The drafter sees the ground-truth prefix
// (teacher forcing).  Each loss is the plain definition, computed in fp64
// from the widened inputs; the L1 distance is summed directly, not through c*.
#include <cmath>
#include <vector>

#include "oracle.h"
#include "oracle_internal.h"

std::vector<double> orc_internal_draft_logits(int V, int r, int dt, double temp,
                                              const void *U_row, const void *W1,
                                              const void *W2, int prev);

static std::vector<double> softmax(const std::vector<double> &z) {
  double m, S;
  orc_internal_stats(z, &m, &S);
  std::vector<double> p(z.size());
  for (size_t v = 0; v < z.size(); ++v) p[v] = std::exp(z[v] - m) / S;
  return p;
}

extern "C" int orc_train_losses(int R, int gamma, int V, int r, int dt, double temp,
                                const void *U, const void *W1, const void *W2, const int32_t *x0,
                                const int32_t *y, const void *P, const float *c, double a_ce,
                                double a_tv, double a_conf, double *per_pos, double *totals) {
  if (R < 1 || gamma < 1 || V < 1 || r < 1 || !(temp > 0.0)) return -1;
  double wsum = 0.0;
  for (int k = 1; k <= gamma; ++k) wsum += std::exp(-(double)(k - 1) / gamma);
  double tot[3] = {0.0, 0.0, 0.0};
  for (int rho = 0; rho < R; ++rho) {
    double req[3] = {0.0, 0.0, 0.0};
    for (int k = 1; k <= gamma; ++k) {
      const int prev = k == 1 ? x0[rho] : y[(size_t)rho * gamma + k - 2];
      const int yk = y[(size_t)rho * gamma + k - 1];
      if (prev < 0 || prev >= V || yk < 0 || yk >= V) return -1;
      const void *U_row = orc_internal_row(dt, U, (int64_t)rho * gamma + k - 1, V);
      const std::vector<double> q =
          softmax(orc_internal_draft_logits(V, r, dt, temp, U_row, W1, W2, prev));
      std::vector<double> t(V);
      const void *P_row = orc_internal_row(dt, P, (int64_t)rho * (gamma + 1) + k - 1, V);
      for (int v = 0; v < V; ++v) t[v] = orc_internal_widen(dt, P_row, v) / temp;
      const std::vector<double> p = softmax(t);
      double l1 = 0.0, cs = 0.0;
      for (int v = 0; v < V; ++v) {
        l1 += std::fabs(p[v] - q[v]);
        cs += std::fmin(p[v], q[v]);
      }
      const double ck = (double)c[(size_t)rho * gamma + k - 1];
      const double ce = -std::log(q[yk]);
      const double bce = -(cs * std::log(ck) + (1.0 - cs) * std::log(1.0 - ck));
      const double w = std::exp(-(double)(k - 1) / gamma);
      const double vals[3] = {ce, l1, bce};
      for (int i = 0; i < 3; ++i) {
        if (per_pos) per_pos[((size_t)i * R + rho) * gamma + k - 1] = vals[i];
        req[i] += w * vals[i];
      }
    }
    for (int i = 0; i < 3; ++i) tot[i] += req[i] / wsum;
  }
  for (int i = 0; i < 3; ++i) totals[i] = tot[i] / R;
  totals[3] = a_ce * totals[0] + a_tv * totals[1] + a_conf * totals[2];
  return 0;
}
