// Forward-only training reductions of the drafter (Blog, "Training
// objective"; KB section 5): on the ground-truth prefix, per position k
//   CE_k   = -log q_k(y_k)                      hard cross-entropy
//   L1_k   = sum_v |p_k(v) - q_k(v)| = 2 (1 - c*_k)   (twice the total variation)
//   BCE_k  = -(c*_k log c_k + (1 - c*_k) log(1 - c_k))  confidence vs soft c*
// weighted by w_k = exp(-(k - 1) / gamma), normalised per request, averaged
// over requests, and combined as a_ce L_ce + a_tv L_tv + a_conf L_conf.
//
// Three launches reuse the hot path itself:
//  1. the draft product + sampler with teacher forcing: x_k is the label
//     y_k, so q_k(y_k) comes out as log q with the draft's exact arithmetic,
//     and step k + 1 conditions on W1[y_k];
//  2. verification with every position admitted (ell = gamma, request rho's
//     rows at rho (gamma + 1)): its sum min(p, q) is c*_k;
//  3. loss_reduce_kernel: one workgroup folds the R x gamma positions in a
//     fixed order (fp64 sums, so the totals do not depend on the schedule).
#include "kernels.h"
#include "common.h"
#include "trace.h"

namespace dspark {

__global__ void train_rows_kernel(int R, int gamma, int32_t *ell, int32_t *row_offset) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i <= R) row_offset[i] = i * (gamma + 1);
  if (i < R) ell[i] = gamma;
}

struct LossParams {
  int R, gamma;
  const float *logq;    // [R][gamma] log q_k(y_k)
  const float *c_star;  // [R][gamma]
  const float *c;       // [R][gamma] confidences
  double a_ce, a_tv, a_conf;
  float *per_pos;       // [3][R][gamma] or NULL
  double *totals;       // [4]
};

constexpr int kLossWaves = 16;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// wave w takes requests w, w + 16, ...; lane k - 1 takes position k
__global__ __launch_bounds__(kLossWaves * kWave) void loss_reduce_kernel(LossParams p) {
  __shared__ double part[kLossWaves][3];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int gamma = p.gamma, k = lane + 1;
  const double wk = k <= gamma ? exp(-(double)(k - 1) / gamma) : 0.0;
  const double wsum = wave_sum_f64(wk);
  double acc[3] = {0.0, 0.0, 0.0};
  for (int rho = wave; rho < p.R; rho += kLossWaves) {
    double v[3] = {0.0, 0.0, 0.0};
    if (k <= gamma) {
      const int64_t s = (int64_t)rho * gamma + lane;
      const double cs = p.c_star[s], ck = p.c[s];
      v[0] = -(double)p.logq[s];
      v[1] = 2.0 * (1.0 - cs);
      v[2] = -(cs * log(ck) + (1.0 - cs) * log(1.0 - ck));
      if (p.per_pos != nullptr) {
        const int64_t n = (int64_t)p.R * gamma;
        p.per_pos[s] = (float)v[0];
        p.per_pos[n + s] = (float)v[1];
        p.per_pos[2 * n + s] = (float)v[2];
      }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) acc[i] += wave_sum_f64(wk * v[i]) / wsum;
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) part[wave][i] = acc[i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t[3] = {0.0, 0.0, 0.0};
    for (int w = 0; w < kLossWaves; ++w)
      for (int i = 0; i < 3; ++i) t[i] += part[w][i];
    for (int i = 0; i < 3; ++i) p.totals[i] = t[i] / p.R;
    p.totals[3] = p.a_ce * (t[0] / p.R) + p.a_tv * (t[1] / p.R) + p.a_conf * (t[2] / p.R);
  }
}

hipError_t launch_train(const TrainLaunch &L, hipStream_t stream) {
  DSPARK_LAUNCH("train_rows", stream, train_rows_kernel, (L.R + 256) / 256, 256, L.R, L.gamma,
                L.ell, L.row_offset);
  hipError_t e = launch_draft(L.draft, stream);
  if (e != hipSuccess) return e;
  e = launch_verify(L.verify, stream);
  if (e != hipSuccess) return e;
  LossParams lp{};
  lp.R = L.R; lp.gamma = L.gamma; lp.logq = L.draft.logq_x; lp.c_star = L.verify.c_star;
  lp.c = L.c; lp.a_ce = L.a_ce; lp.a_tv = L.a_tv; lp.a_conf = L.a_conf;
  lp.per_pos = L.per_pos; lp.totals = L.totals;
  DSPARK_LAUNCH("loss_reduce", stream, loss_reduce_kernel, 1, kLossWaves * kWave, lp);
  return hipGetLastError();
}

}  // namespace dspark
