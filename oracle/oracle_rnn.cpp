// DSpark hot path, CPU oracle: the recurrent sequential head's state.  TEST
// INFRASTRUCTURE ONLY (see oracle.h).
//
// Blog, "RNN sequential head": instead of the previous token alone, the head
// carries a small running state s_k = f(s_{k-1}, E(x_{k-1}), h_k) and adds
// W_o s_k to the block logits.  KB section 3: the state, the previous token's
// embedding and the position's backbone hidden state are concatenated and
// combined by a gated update.  The gated update is read as the standard gated
// recurrent unit (Cho et al., 2014), written out in fp64 from the widened inputs.
#include <cmath>
#include <vector>

#include "oracle.h"
#include "oracle_internal.h"

static double sigmoid(double t) { return 1.0 / (1.0 + std::exp(-t)); }

extern "C" int orc_rnn_states(int gamma, int V, int r, int dt, const void *G_E,
                              const float *G_h, const void *W_hh, const float *b_hh, int x0,
                              const int32_t *x, const float *s0, double *s_out) {
  if (gamma < 1 || V < 1 || r < 1 || !G_E || !G_h || !W_hh || !b_hh || !s_out) return -1;
  const int g3 = 3 * r;
  std::vector<double> s(r, 0.0), a(g3), g(g3);
  if (s0)
    for (int i = 0; i < r; ++i) s[i] = s0[i];
  for (int k = 1; k <= gamma; ++k) {
    const int prev = k == 1 ? x0 : x[k - 2];
    if (prev < 0 || prev >= V) return -1;
    for (int j = 0; j < g3; ++j) {
      g[j] = orc_internal_widen(dt, G_E, (int64_t)prev * g3 + j) + (double)G_h[(k - 1) * g3 + j];
      double acc = b_hh[j];
      for (int i = 0; i < r; ++i) acc += orc_internal_widen(dt, W_hh, (int64_t)i * g3 + j) * s[i];
      a[j] = acc;
    }
    std::vector<double> next(r);
    for (int j = 0; j < r; ++j) {
      const double rg = sigmoid(g[j] + a[j]);
      const double zg = sigmoid(g[r + j] + a[r + j]);
      const double n = std::tanh(g[2 * r + j] + rg * a[2 * r + j]);
      next[j] = (1.0 - zg) * n + zg * s[j];
    }
    s = next;
    for (int j = 0; j < r; ++j) s_out[(size_t)(k - 1) * r + j] = s[j];
  }
  return 0;
}
