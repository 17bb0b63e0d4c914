// DSpark hot path, CPU oracle: random numbers, element widening, softmax
// statistics, inverse CDF, TV overlap.  TEST INFRASTRUCTURE ONLY (see oracle.h).
#include "oracle.h"

#include <cmath>
#include <cstring>
#include <vector>

// ---------------------------------------------------------------------------
// Philox4x64-10, from the definition in Salmon et al., SC'11.  One round maps
// (X0, X1, X2, X3) with key (K0, K1) to
//   (hi(M1*X2) ^ X1 ^ K0, lo(M1*X2), hi(M0*X0) ^ X3 ^ K1, lo(M0*X0));
// between rounds the key is bumped by the Weyl constants (golden ratio and
// sqrt(3) - 1, as 64-bit fractions).
// ---------------------------------------------------------------------------
static const uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ULL;
static const uint64_t kPhiloxM1 = 0xCA5A826395121157ULL;
static const uint64_t kWeyl0 = 0x9E3779B97F4A7C15ULL;
static const uint64_t kWeyl1 = 0xBB67AE8584CAA73BULL;

static void mul_hi_lo(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo) {
  unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

extern "C" void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += kWeyl0;
      k1 += kWeyl1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mul_hi_lo(kPhiloxM0, x0, &hi0, &lo0);
    mul_hi_lo(kPhiloxM1, x2, &hi1, &lo1);
    uint64_t n0 = hi1 ^ x1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ x3 ^ k1;
    uint64_t n3 = lo0;
    x0 = n0; x1 = n1; x2 = n2; x3 = n3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

extern "C" double orc_uniform(uint64_t seed, uint64_t round, uint64_t pos, uint64_t req,
                              uint64_t stream) {
  const uint64_t ctr[4] = {pos, req, stream, round};
  const uint64_t key[2] = {seed, 0};
  uint64_t out[4];
  orc_philox4x64_10(ctr, key, out);
  // top 24 bits of the first word, as a multiple of 2^-24
  return (double)(out[0] >> 40) * (1.0 / 16777216.0);
}

// ---------------------------------------------------------------------------
// Element widening.  bfloat16 is the high half of a binary32, so the widening
// is exact; binary32 to binary64 is exact too.
// ---------------------------------------------------------------------------
static double widen_one(int dt, const void *src, int64_t i) {
  if (dt == ORC_F32) return (double)((const float *)src)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)src)[i] << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return (double)f;
}

extern "C" void orc_widen(int dt, const void *src, int64_t n, double *dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = widen_one(dt, src, i);
}

static int64_t elem_size(int dt) { return dt == ORC_F32 ? 4 : 2; }

static const void *row_ptr(int dt, const void *base, int64_t row, int64_t len) {
  return (const char *)base + row * len * elem_size(dt);
}

// ---------------------------------------------------------------------------
// Softmax statistics: m = max z, S = sum_v e^{z_v - m}, z = x / T.
// ---------------------------------------------------------------------------
static void stats_of(const std::vector<double> &z, double *m, double *S) {
  double mx = -INFINITY;
  for (double v : z) mx = v > mx ? v : mx;
  double s = 0.0;
  for (double v : z) s += std::exp(v - mx);
  *m = mx;
  *S = s;
}

static std::vector<double> scaled_row(int V, int dt, double temp, const void *row) {
  std::vector<double> z(V);
  for (int v = 0; v < V; ++v) z[v] = widen_one(dt, row, v) / temp;
  return z;
}

extern "C" int orc_row_stats(int V, int dt, double temp, const void *row, double *m, double *S) {
  if (V < 1) return -1;
  std::vector<double> z = scaled_row(V, dt, temp, row);
  stats_of(z, m, S);
  return 0;
}

static std::vector<double> softmax_of(const std::vector<double> &z) {
  double m, S;
  stats_of(z, &m, &S);
  std::vector<double> p(z.size());
  for (size_t v = 0; v < z.size(); ++v) p[v] = std::exp(z[v] - m) / S;
  return p;
}

// ---------------------------------------------------------------------------
// Inverse CDF on non-negative masses.
// ---------------------------------------------------------------------------
extern "C" int orc_inverse_cdf(int V, const double *w, double u, double *cdf) {
  double total = 0.0;
  for (int v = 0; v < V; ++v) total += w[v];
  if (!(total > 0.0)) return -1;
  const double target = u * total;
  int pick = -1, last_positive = -1;
  double run = 0.0;
  for (int v = 0; v < V; ++v) {
    run += w[v];
    if (w[v] > 0.0) last_positive = v;
    if (cdf) cdf[v] = run / total;
    if (pick < 0 && target < run) pick = v;
  }
  return pick >= 0 ? pick : last_positive;
}

// ---------------------------------------------------------------------------
// TV overlap label: c* = sum_v min(p, q); also 1/2 ||p - q||_1 for the identity
// c* = 1 - TV (Blog "Total variation label", "Coupling view").
// ---------------------------------------------------------------------------
extern "C" double orc_overlap(int V, int dt, double temp, const void *P_row, const void *Q_row,
                              double *tv) {
  std::vector<double> p = softmax_of(scaled_row(V, dt, temp, P_row));
  std::vector<double> q = softmax_of(scaled_row(V, dt, temp, Q_row));
  double overlap = 0.0, l1 = 0.0;
  for (int v = 0; v < V; ++v) {
    overlap += std::fmin(p[v], q[v]);
    l1 += std::fabs(p[v] - q[v]);
  }
  if (tv) *tv = 0.5 * l1;
  return overlap;
}

// Shared with the draft and verify translation units of the oracle.
double orc_internal_widen(int dt, const void *src, int64_t i) { return widen_one(dt, src, i); }
const void *orc_internal_row(int dt, const void *base, int64_t row, int64_t len) {
  return row_ptr(dt, base, row, len);
}
std::vector<double> orc_internal_softmax(const std::vector<double> &z) { return softmax_of(z); }
void orc_internal_stats(const std::vector<double> &z, double *m, double *S) { stats_of(z, m, S); }
std::vector<double> orc_internal_scaled_row(int V, int dt, double temp, const void *row) {
  return scaled_row(V, dt, temp, row);
}
