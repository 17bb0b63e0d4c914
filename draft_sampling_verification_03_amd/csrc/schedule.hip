// Hardware-aware prefix scheduler (KB section 4; Blog "Scheduler objective",
// "Greedy prefix allocation", "Async scheduler in practice"; Bangkok 4.2.2;
// Reaper 3.3) in one workgroup of 1024 threads.
//
//  1. survival a[rho][j] = fl32(a[rho][j-1] * c[rho][j]), one thread per request,
//     left to right (binary32, as the products that rank the candidates)
//  2. candidate keys ((0xFFFFFFFF - bits(a)) << 32) | (j << 20) | rho: ascending
//     key order is a descending, then depth ascending, then request ascending;
//     a >= 0 so its bit pattern orders like its value.  Bitonic sort in LDS.
//  3. fixed-point path A_n = sum of floor(a_(i) 2^32) (int64, exact in any
//     order), tau_n = R + A_n 2^-32, theta_n = tau_n * SPS[R + n] (fp64)
//  4. n* by mode; ell[rho] = number of rho's keys <= the n*-th key (keys along
//     one request increase with depth, so this counts an admitted prefix);
//     row_offset = exclusive scan of 1 + ell.
#include <float.h>
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kMaxCandidates = 8192;

struct SchedShared {
  uint64_t keys[kMaxCandidates];
  float conf[kMaxCandidates];  // the confidences being ranked, staged from global memory
  int64_t wave_i64[kSchedWaves];
  double wave_d[kSchedWaves];
  int wave_i[kSchedWaves];
  int flag;
};

__device__ __forceinline__ float survival_step(float run, float c, int32_t *err, bool *bad) {
  if (!(c >= 0.0f && c <= 1.0f)) {  // also NaN
    *bad = true;
    c = 0.0f;
  }
  (void)err;
  return run * c;
}

// c -> sh.conf with every load of a thread in flight at once (coalesced)
__device__ __forceinline__ void stage_confidences(const float *c, int N, SchedShared &sh) {
  constexpr int kIt = kMaxCandidates / kSchedThreads;
  float v[kIt];
#pragma unroll
  for (int j = 0; j < kIt; ++j) {
    const int i = threadIdx.x + j * kSchedThreads;
    v[j] = i < N ? c[i] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kIt; ++j) {
    const int i = threadIdx.x + j * kSchedThreads;
    if (i < N) sh.conf[i] = v[j];
  }
  __syncthreads();
}

__device__ __forceinline__ uint64_t cand_key(float a, int j, int rho) {
  return ((uint64_t)(0xFFFFFFFFu - __float_as_uint(a)) << 32) | ((uint64_t)j << 20) | (uint64_t)rho;
}
__device__ __forceinline__ float key_a(uint64_t key) {
  return __uint_as_float(0xFFFFFFFFu - (uint32_t)(key >> 32));
}
__device__ __forceinline__ int64_t fixed_weight(float a) {
  return (int64_t)((double)a * 4294967296.0);  // a in [0, 1]: exact product, truncation = floor
}

// exclusive scan of int64 over the workgroup (thread order); returns the prefix
__device__ int64_t sched_exclusive_scan_i64(int64_t v, SchedShared &sh, int64_t *total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int64_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == kWave - 1) sh.wave_i64[w] = inc;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int i = 0; i < kSchedWaves; ++i) {
    if (i < w) before += sh.wave_i64[i];
    all += sh.wave_i64[i];
  }
  *total = all;
  __syncthreads();
  return before + inc - v;
}

__device__ int sched_min_int(int v, SchedShared &sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_min_int(v);
  __syncthreads();
  if (lane == 0) sh.wave_i[w] = v;
  __syncthreads();
  int r = sh.wave_i[0];
  for (int i = 1; i < kSchedWaves; ++i) r = min(r, sh.wave_i[i]);
  __syncthreads();
  return r;
}

// (theta, n) maximum with the smallest n among equal theta
__device__ void sched_argmax(double *th, int *n, SchedShared &sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  double t = *th;
  int m = *n;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double t2 = __shfl_xor(t, o);
    const int m2 = __shfl_xor(m, o);
    if (t2 > t || (t2 == t && m2 < m)) {
      t = t2;
      m = m2;
    }
  }
  __syncthreads();
  if (lane == 0) {
    sh.wave_d[w] = t;
    sh.wave_i[w] = m;
  }
  __syncthreads();
  t = sh.wave_d[0];
  m = sh.wave_i[0];
  for (int i = 1; i < kSchedWaves; ++i)
    if (sh.wave_d[i] > t || (sh.wave_d[i] == t && sh.wave_i[i] < m)) {
      t = sh.wave_d[i];
      m = sh.wave_i[i];
    }
  __syncthreads();
  *th = t;
  *n = m;
}

// Sort the candidates of confidences c into sh.keys (ascending); returns N.
// Writes a when a_out is not NULL.
__device__ int sorted_candidates(int R, int gamma, const float *c, float *a_out, int32_t *err,
                                 SchedShared &sh) {
  const int N = R * gamma;
  int P2 = 1;
  while (P2 < N) P2 <<= 1;
  stage_confidences(c, N, sh);
  bool bad = false;
  for (int rho = threadIdx.x; rho < R; rho += kSchedThreads) {
    float run = 1.0f;
    for (int j = 1; j <= gamma; ++j) {
      const int64_t idx = (int64_t)rho * gamma + (j - 1);
      run = survival_step(run, sh.conf[idx], err, &bad);
      if (a_out) a_out[idx] = run;
      sh.keys[idx] = cand_key(run, j, rho);
    }
  }
  if (bad) flag_error(err, kErrConfidence);
  for (int i = N + threadIdx.x; i < P2; i += kSchedThreads) sh.keys[i] = ~(uint64_t)0;
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int idx = threadIdx.x; idx < (P2 >> 1); idx += kSchedThreads) {
        const int i = 2 * idx - (idx & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t x = sh.keys[i], y = sh.keys[j];
        if ((x > y) == up) {
          sh.keys[i] = y;
          sh.keys[j] = x;
        }
      }
      __syncthreads();
    }
  }
  return N;
}

// Walk the sorted path; returns n* for EARLY_STOP or FULL_SEARCH and theta_{n*}.
__device__ int select_on_path(int R, int N, int mode, const double *SPS, SchedShared &sh,
                              double *theta_star) {
  const int cpt = (N + kSchedThreads - 1) / kSchedThreads;
  const int i0 = min((int)threadIdx.x * cpt, N), i1 = min(i0 + cpt, N);
  int64_t local = 0;
  for (int i = i0; i < i1; ++i) local += fixed_weight(key_a(sh.keys[i]));
  int64_t total;
  const int64_t base = sched_exclusive_scan_i64(local, sh, &total);
  // theta_n for n = i + 1 (after admitting sorted candidate i); theta_0 apart
  const double inv32 = 1.0 / 4294967296.0;
  const double theta0 = (double)R * SPS[R];
  int n_star;
  if (mode == 1) {  // EARLY_STOP: first n with !(theta_{n+1} > theta_n)
    int cand = 0x7fffffff;
    int64_t A = base;
    double prev = i0 == 0 ? theta0 : ((double)R + (double)base * inv32) * SPS[R + i0];
    for (int i = i0; i < i1; ++i) {
      A += fixed_weight(key_a(sh.keys[i]));
      const double th = ((double)R + (double)A * inv32) * SPS[R + i + 1];
      if (cand == 0x7fffffff && !(th > prev)) cand = i;  // n = i fails to grow
      prev = th;
    }
    n_star = sched_min_int(cand, sh);
    if (n_star == 0x7fffffff) n_star = N;
  } else {  // FULL_SEARCH: smallest argmax over n = 0..N
    double best = threadIdx.x == 0 ? theta0 : -INFINITY;
    int best_n = threadIdx.x == 0 ? 0 : 0x7fffffff;
    int64_t A = base;
    for (int i = i0; i < i1; ++i) {
      A += fixed_weight(key_a(sh.keys[i]));
      const double th = ((double)R + (double)A * inv32) * SPS[R + i + 1];
      if (th > best) {
        best = th;
        best_n = i + 1;
      }
    }
    sched_argmax(&best, &best_n, sh);
    n_star = best_n;
  }
  // theta at n*: the thread whose chunk ends at n* (or theta_0)
  if (n_star == 0) {
    if (threadIdx.x == 0) *theta_star = theta0;
  } else if (i0 < n_star && n_star <= i1) {
    int64_t A = base;
    for (int i = i0; i < n_star; ++i) A += fixed_weight(key_a(sh.keys[i]));
    *theta_star = ((double)R + (double)A * inv32) * SPS[R + n_star];
  }
  return n_star;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleLaunch L) {
  __shared__ SchedShared sh;
  __shared__ double s_theta;
  const int R = L.R, gamma = L.gamma, N = R * gamma;
  int n_star = N;
  if (threadIdx.x == 0) s_theta = NAN;
  __syncthreads();

  uint64_t threshold = ~(uint64_t)0;  // OFF: everything admitted
  if (L.mode == 0) {
    if (L.c != nullptr) {
      stage_confidences(L.c, N, sh);
      bool bad = false;
      int64_t local = 0;
      for (int rho = threadIdx.x; rho < R; rho += kSchedThreads) {
        float run = 1.0f;
        for (int j = 1; j <= gamma; ++j) {
          const int64_t idx = (int64_t)rho * gamma + (j - 1);
          run = survival_step(run, sh.conf[idx], L.err, &bad);
          if (L.a) L.a[idx] = run;
          local += fixed_weight(run);
        }
      }
      if (bad) flag_error(L.err, kErrConfidence);
      int64_t total;
      sched_exclusive_scan_i64(local, sh, &total);
      if (threadIdx.x == 0 && L.SPS != nullptr)
        s_theta = ((double)R + (double)total * (1.0 / 4294967296.0)) * L.SPS[R + N];
    }
  } else {
    double theta_star = NAN;
    if (L.mode == 3) {  // capacity from round t-2, by full search on its own path
      sorted_candidates(R, gamma, L.c_prev2, nullptr, L.err, sh);
      double unused = 0.0;
      n_star = select_on_path(R, N, 2, L.SPS, sh, &unused);
      __syncthreads();
    }
    sorted_candidates(R, gamma, L.c, L.a, L.err, sh);
    if (L.mode == 3) {
      // theta of the top n_star current candidates
      const int cpt = (N + kSchedThreads - 1) / kSchedThreads;
      const int i0 = min((int)threadIdx.x * cpt, N), i1 = min(i0 + cpt, N);
      int64_t local = 0;
      for (int i = i0; i < i1 && i < n_star; ++i) local += fixed_weight(key_a(sh.keys[i]));
      int64_t total;
      sched_exclusive_scan_i64(local, sh, &total);
      if (threadIdx.x == 0) theta_star = ((double)R + (double)total * (1.0 / 4294967296.0)) * L.SPS[R + n_star];
    } else {
      n_star = select_on_path(R, N, L.mode, L.SPS, sh, &theta_star);
    }
    __syncthreads();
    if (!isnan(theta_star)) s_theta = theta_star;  // exactly one thread holds it
    threshold = n_star > 0 ? sh.keys[n_star - 1] : 0;
  }
  __syncthreads();

  // lengths: count each request's keys <= threshold (a prefix), then offsets
  // (sh.conf holds the current confidences: the last array staged)
  constexpr int kMaxPerThread = kMaxCandidates / kSchedThreads;  // R <= N <= 8192
  const int cpr = (R + kSchedThreads - 1) / kSchedThreads;
  const int r0 = min((int)threadIdx.x * cpr, R), r1 = min(r0 + cpr, R);
  int lens[kMaxPerThread];
  int64_t local = 0;
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int rho = r0 + q;
    lens[q] = 0;
    if (rho < r1) {
      int l = gamma;
      if (L.mode != 0) {
        bool bad = false;
        float run = 1.0f;
        l = 0;
        for (int j = 1; j <= gamma; ++j) {
          run = survival_step(run, sh.conf[(int64_t)rho * gamma + (j - 1)], L.err, &bad);
          if (cand_key(run, j, rho) <= threshold && n_star > 0) l = j; else break;
        }
      }
      L.ell[rho] = l;
      lens[q] = l;
      local += 1 + l;
    }
  }
  int64_t total;
  int64_t off = sched_exclusive_scan_i64(local, sh, &total);
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int rho = r0 + q;
    if (rho < r1) {
      L.row_offset[rho] = (int32_t)off;
      off += 1 + lens[q];
    }
  }
  if (threadIdx.x == 0) {
    L.row_offset[R] = (int32_t)total;
    *L.n_admitted = n_star;
    *L.theta = s_theta;
  }
}

hipError_t launch_schedule(const ScheduleLaunch &L, hipStream_t stream) {
  DSPARK_LAUNCH("schedule", stream, schedule_kernel<<<1, kSchedThreads, 0, stream>>>(L));
  return hipGetLastError();
}

}  // namespace dspark
