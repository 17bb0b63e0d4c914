// DSpark hot path, CPU oracle: the hardware-aware prefix scheduler.
// TEST INFRASTRUCTURE ONLY (see oracle.h).
//
// KB section 4 states the problem: choose ell_rho per request; the target batch
// is B = sum_rho (1 + ell_rho), the expected committed tokens
// tau = sum_rho (1 + sum_{j <= ell_rho} a_{rho,j}) with a_{rho,j} = prod_{i<=j} c_{rho,i},
// and the objective is theta = tau * SPS(B) against a table profiled at start-up.
// Blog "Greedy prefix allocation" and Reaper 3.3: sort every (request, depth)
// candidate by a and admit along that order; monotone a keeps each request's
// admitted set a prefix.  Stop rule (KB section 4, Bangkok 4.2.2): the ideal
// scheduler stops the first time theta does not increase; with a stepped SPS
// the production scheduler searches the whole path; with the async variant the
// capacity K comes from confidences two rounds old and the current scores fill
// the K slots (Blog "Async scheduler in practice").
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "oracle.h"

namespace {

struct Candidate {
  float a;
  int j;    // depth, 1-based
  int rho;  // request
};

// Survival products in binary32, left to right: a_j = fl32(a_{j-1} * c_j).
// A confidence is a probability: -0.0 is the value 0 and is read as +0.0, so
// every survival product is a non-negative number with a non-negative sign.
bool survival(int R, int gamma, const float *c, std::vector<float> &a) {
  a.assign((size_t)R * gamma, 0.0f);
  for (int rho = 0; rho < R; ++rho) {
    float run = 1.0f;
    for (int j = 1; j <= gamma; ++j) {
      float cj = c[(size_t)rho * gamma + (j - 1)];
      if (!(cj >= 0.0f && cj <= 1.0f)) return false;  // also rejects NaN
      if (cj == 0.0f) cj = 0.0f;                        // -0.0 -> +0.0
      run = run * cj;
      a[(size_t)rho * gamma + (j - 1)] = run;
    }
  }
  return true;
}

// Global order: a descending, then depth ascending, then request ascending.
std::vector<Candidate> sorted_candidates(int R, int gamma, const std::vector<float> &a) {
  std::vector<Candidate> cand;
  cand.reserve((size_t)R * gamma);
  for (int rho = 0; rho < R; ++rho)
    for (int j = 1; j <= gamma; ++j) cand.push_back({a[(size_t)rho * gamma + (j - 1)], j, rho});
  std::sort(cand.begin(), cand.end(), [](const Candidate &x, const Candidate &y) {
    if (x.a != y.a) return x.a > y.a;
    if (x.j != y.j) return x.j < y.j;
    return x.rho < y.rho;
  });
  return cand;
}

// Fixed-point weight of one candidate: floor(a * 2^32), exact for a in [0, 1].
int64_t fixed_weight(float a) { return (int64_t)std::floor((double)a * 4294967296.0); }

// theta_n for n = 0..N along the sorted path (fixed-point tau).
std::vector<double> theta_path(int R, const std::vector<Candidate> &cand, const double *SPS) {
  const int N = (int)cand.size();
  std::vector<double> theta(N + 1);
  int64_t A = 0;
  for (int n = 0; n <= N; ++n) {
    if (n > 0) A += fixed_weight(cand[n - 1].a);
    const double tau = (double)R + (double)A * (1.0 / 4294967296.0);
    theta[n] = tau * SPS[R + n];
  }
  return theta;
}

// The same path with a plain fp64 running sum of a (diagnostic).
std::vector<double> theta_path_plain(int R, const std::vector<Candidate> &cand,
                                     const double *SPS) {
  const int N = (int)cand.size();
  std::vector<double> theta(N + 1);
  double tau = (double)R;
  for (int n = 0; n <= N; ++n) {
    if (n > 0) tau += (double)cand[n - 1].a;
    theta[n] = tau * SPS[R + n];
  }
  return theta;
}

}  // namespace

extern "C" int orc_select_n(const double *theta, int N, int mode) {
  if (mode == ORC_SCHED_EARLY_STOP) {
    int n = 0;
    while (n < N && theta[n + 1] > theta[n]) ++n;  // admit only on a strict increase
    return n;
  }
  if (mode == ORC_SCHED_FULL_SEARCH) {
    int best = 0;
    for (int n = 1; n <= N; ++n)
      if (theta[n] > theta[best]) best = n;  // strict: the smallest maximizer wins
    return best;
  }
  return -1;
}

extern "C" int orc_schedule(int R, int gamma, int mode, double threshold, const float *c,
                            const float *c_prev2,
                            const double *SPS, int B_max, int32_t *ell, int32_t *row_offset,
                            float *a_out, int32_t *n_admitted, double *theta, int32_t *n_plain,
                            double *theta_plain) {
  if (R < 1 || gamma < 1) return -1;
  const int N = R * gamma;
  if (mode == ORC_SCHED_THRESHOLD) {
    if (!c || !std::isfinite(threshold)) return -1;
    if (SPS && B_max < R + N) return -1;
    std::vector<float> a;
    if (!survival(R, gamma, c, a)) return -1;
    if (a_out) std::memcpy(a_out, a.data(), sizeof(float) * (size_t)N);
    int n = 0;
    int64_t A = 0;
    double A_plain = 0.0;
    row_offset[0] = 0;
    for (int rho = 0; rho < R; ++rho) {
      int l = 0;
      while (l < gamma && (double)c[(size_t)rho * gamma + l] >= threshold) {
        A += fixed_weight(a[(size_t)rho * gamma + l]);
        A_plain += (double)a[(size_t)rho * gamma + l];
        ++l;
      }
      ell[rho] = l;
      n += l;
      row_offset[rho + 1] = row_offset[rho] + 1 + l;
    }
    *n_admitted = n;
    *theta = SPS ? ((double)R + (double)A * 0x1p-32) * SPS[R + n] : NAN;
    if (n_plain) *n_plain = n;
    if (theta_plain) *theta_plain = SPS ? ((double)R + A_plain) * SPS[R + n] : NAN;
    return 0;
  }
  if (mode < ORC_SCHED_OFF || mode > ORC_SCHED_ASYNC_TOPK) return -1;
  if (mode != ORC_SCHED_OFF && (!c || !SPS || B_max < R + N)) return -1;
  if (mode == ORC_SCHED_ASYNC_TOPK && !c_prev2) return -1;

  std::vector<float> a;
  std::vector<Candidate> cand;
  std::vector<double> th, th_plain;
  const bool have_c = c != nullptr && SPS != nullptr && B_max >= R + N;
  if (have_c) {
    if (!survival(R, gamma, c, a)) return -1;
    cand = sorted_candidates(R, gamma, a);
    th = theta_path(R, cand, SPS);
    th_plain = theta_path_plain(R, cand, SPS);
    if (a_out) std::memcpy(a_out, a.data(), sizeof(float) * (size_t)N);
  }

  int n_star = N, n_star_plain = N;
  if (mode == ORC_SCHED_EARLY_STOP || mode == ORC_SCHED_FULL_SEARCH) {
    n_star = orc_select_n(th.data(), N, mode);
    n_star_plain = orc_select_n(th_plain.data(), N, mode);
  } else if (mode == ORC_SCHED_ASYNC_TOPK) {
    // capacity from the older confidences, by full search on their own path
    std::vector<float> a_old;
    if (!survival(R, gamma, c_prev2, a_old)) return -1;
    std::vector<Candidate> cand_old = sorted_candidates(R, gamma, a_old);
    const int K = orc_select_n(theta_path(R, cand_old, SPS).data(), N, ORC_SCHED_FULL_SEARCH);
    const int K_plain =
        orc_select_n(theta_path_plain(R, cand_old, SPS).data(), N, ORC_SCHED_FULL_SEARCH);
    n_star = K;
    n_star_plain = K_plain;
  }

  for (int rho = 0; rho < R; ++rho) ell[rho] = mode == ORC_SCHED_OFF ? gamma : 0;
  if (mode != ORC_SCHED_OFF)
    for (int i = 0; i < n_star; ++i) ell[cand[i].rho] += 1;  // prefix-closed by the order
  row_offset[0] = 0;
  for (int rho = 0; rho < R; ++rho) row_offset[rho + 1] = row_offset[rho] + 1 + ell[rho];
  *n_admitted = n_star;
  *theta = have_c ? th[n_star] : NAN;
  if (n_plain) *n_plain = n_star_plain;
  if (theta_plain) *theta_plain = have_c ? th_plain[n_star_plain] : NAN;
  return 0;
}

extern "C" double orc_schedule_bruteforce(int R, int gamma, const float *c, const double *SPS,
                                          int B_max, int32_t *ell_best) {
  std::vector<float> a;
  if (R < 1 || gamma < 1 || B_max < R * (1 + gamma) || !survival(R, gamma, c, a)) return NAN;
  // weight of admitting depths 1..l of request rho, fixed point
  std::vector<int64_t> prefix((size_t)R * (gamma + 1), 0);
  for (int rho = 0; rho < R; ++rho)
    for (int j = 1; j <= gamma; ++j)
      prefix[(size_t)rho * (gamma + 1) + j] =
          prefix[(size_t)rho * (gamma + 1) + j - 1] + fixed_weight(a[(size_t)rho * gamma + j - 1]);
  std::vector<int> l(R, 0);
  double best = -INFINITY;
  int best_total = 0;
  while (true) {
    int64_t A = 0;
    int total = 0;
    for (int rho = 0; rho < R; ++rho) {
      A += prefix[(size_t)rho * (gamma + 1) + l[rho]];
      total += l[rho];
    }
    const double th = ((double)R + (double)A * (1.0 / 4294967296.0)) * SPS[R + total];
    if (th > best || (th == best && total < best_total)) {
      best = th;
      best_total = total;
      if (ell_best)
        for (int rho = 0; rho < R; ++rho) ell_best[rho] = l[rho];
    }
    int pos = 0;  // odometer over [0, gamma]^R
    while (pos < R && l[pos] == gamma) l[pos++] = 0;
    if (pos == R) break;
    ++l[pos];
  }
  return best;
}
