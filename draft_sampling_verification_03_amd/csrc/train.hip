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
//  3. loss_request_kernel (one wave per request: the positions' losses and
//     the request's weighted means) and loss_fold_kernel (one workgroup
//     folds the request means in a fixed order; fp64 sums, so the totals do
//     not depend on the schedule).
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
  double *req_sums;     // [R][3]
  double *totals;       // [4]
};

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per request (lane k - 1 takes position k): the position's
// (CE, L1, BCE) and the request's position-weighted means.
__global__ __launch_bounds__(kBlock) void loss_request_kernel(LossParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int rho = blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (rho >= p.R) return;
  const int gamma = p.gamma, k = lane + 1;
  const double wk = k <= gamma ? exp(-(double)(k - 1) / gamma) : 0.0;
  const double wsum = wave_sum_f64(wk);
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
  for (int i = 0; i < 3; ++i) {
    const double m = wave_sum_f64(wk * v[i]) / wsum;
    if (lane == 0) p.req_sums[(int64_t)rho * 3 + i] = m;
  }
}

// The request means folded in a fixed order: thread t sums requests t,
// t + kBlock, ... in turn, then thread 0 the threads' sums in thread order.
__global__ __launch_bounds__(kBlock) void loss_fold_kernel(LossParams p) {
  __shared__ double part[kBlock][3];
  const int t = threadIdx.x;
  double acc[3] = {0.0, 0.0, 0.0};
  for (int rho = t; rho < p.R; rho += kBlock)
#pragma unroll
    for (int i = 0; i < 3; ++i) acc[i] += p.req_sums[(int64_t)rho * 3 + i];
#pragma unroll
  for (int i = 0; i < 3; ++i) part[t][i] = acc[i];
  __syncthreads();
  if (t == 0) {
    double tot[3] = {0.0, 0.0, 0.0};
    for (int w = 0; w < kBlock; ++w)
      for (int i = 0; i < 3; ++i) tot[i] += part[w][i];
    for (int i = 0; i < 3; ++i) p.totals[i] = tot[i] / p.R;
    p.totals[3] = p.a_ce * (tot[0] / p.R) + p.a_tv * (tot[1] / p.R) + p.a_conf * (tot[2] / p.R);
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
  lp.per_pos = L.per_pos; lp.totals = L.totals; lp.req_sums = L.req_sums;
  DSPARK_LAUNCH("loss_request", stream, loss_request_kernel, (L.R + kBlock / kWave - 1) / (kBlock / kWave),
                kBlock, lp);
  DSPARK_LAUNCH("loss_fold", stream, loss_fold_kernel, 1, kBlock, lp);
  return hipGetLastError();
}

}  // namespace dspark
