// Hardware-aware prefix scheduler (KB section 4; Blog "Scheduler objective",
// "Greedy prefix allocation", "Async scheduler in practice"; Bangkok 4.2.2;
// Reaper 3.3) in one workgroup of 1024 threads.
//
//  1. survival a[rho][j] = fl32(a[rho][j-1] * c[rho][j]), one thread per request,
//     left to right (binary32, as the products that rank the candidates)
//  2. candidate keys ((0xFFFFFFFF - bits(a)) << 32) | (j << 20) | rho: ascending
//     key order is a descending, then depth ascending, then request ascending;
//     a >= +0 (a -0.0 confidence is read as +0.0) so its bit pattern orders
//     like its value.  Bitonic sort with the
//     keys in registers (E per thread, blocked): strides inside a thread swap
//     registers, strides inside a wave use lane shuffles, and only strides
//     across waves exchange through LDS (two barriers each).
//  3. fixed-point path A_n = sum of floor(a_(i) 2^32) (int64, exact in any
//     order), tau_n = R + A_n 2^-32, theta_n = tau_n * SPS[R + n] (fp64); the
//     SPS entries a thread needs are loaded before the sort.
//  4. n* by mode; ell[rho] = number of rho's admitted keys (sorted positions
//     < n*; keys along one request increase with depth, so they are a prefix
//     and the count is the deepest admitted j); row_offset = exclusive scan of
//     1 + ell.
#include <float.h>
#include <math.h>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kMaxCandidates = 8192;
// confidences staged with an odd row pitch (gamma | 1): the survival thread of
// request rho reads row rho, and odd pitches keep those reads conflict-free
constexpr int kConfSlots = kMaxCandidates + kMaxCandidates / 2;

struct SchedShared {
  uint64_t keys[kMaxCandidates];  // candidate keys; cross-wave exchange of the sort
  union {
    float conf[kConfSlots];       // confidences, then survival (in place)
    int ell[kMaxCandidates];      // admitted depth per request
    uint64_t keys2[kMaxCandidates];  // second exchange buffer of the sort
  };
  int64_t wave_i64[kSchedWaves];
  double wave_d[kSchedWaves];
  int wave_i[kSchedWaves];
};

__device__ __forceinline__ uint64_t cand_key(float a, int j, int rho) {
  return ((uint64_t)(0xFFFFFFFFu - __float_as_uint(a)) << 32) | ((uint64_t)j << 20) | (uint64_t)rho;
}
__device__ __forceinline__ float key_a(uint64_t key) {
  return __uint_as_float(0xFFFFFFFFu - (uint32_t)(key >> 32));
}
__device__ __forceinline__ int key_j(uint64_t key) { return (int)((key >> 20) & 0xFFF); }
__device__ __forceinline__ int key_rho(uint64_t key) { return (int)(key & 0xFFFFF); }
__device__ __forceinline__ int64_t fixed_weight(float a) {
  return (int64_t)((double)a * 4294967296.0);  // a in [0, 1]: exact product, truncation = floor
}

// exclusive scan of int64 over the workgroup (thread order); returns the prefix
__device__ __forceinline__ int64_t sched_exclusive_scan_i64(int64_t v, SchedShared &sh, int64_t *total) {
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
  return before + inc - v;
}

__device__ __forceinline__ int sched_min_int(int v, SchedShared &sh) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_min_int(v);
  __syncthreads();
  if (lane == 0) sh.wave_i[w] = v;
  __syncthreads();
  int r = sh.wave_i[0];
  for (int i = 1; i < kSchedWaves; ++i) r = min(r, sh.wave_i[i]);
  return r;
}

// (theta, n) maximum with the smallest n among equal theta
__device__ __forceinline__ void sched_argmax(double *th, int *n, SchedShared &sh) {
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
  *th = t;
  *n = m;
}

// c -> sh.conf (row pitch gs) with every load of a thread in flight at once
__device__ __forceinline__ void stage_confidences(const float *c, int N, int gamma, int gs,
                                                  SchedShared &sh) {
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
    if (i < N) {
      const int rho = i / gamma;
      sh.conf[rho * gs + (i - rho * gamma)] = v[j];
    }
  }
  __syncthreads();
}

// Survival a[rho][j] = fl32(a[rho][j-1] c[rho][j]) along each request (one
// thread per request, left to right), in place in sh.conf.  With keys, the
// candidate key of (rho, j) goes to sh.keys[(j - 1) R + rho] (any placement
// works: the sort orders them).  Returns this thread's sum of fixed-point
// weights; flags a confidence outside [0, 1] (or NaN) and uses 0 for it.
__device__ __forceinline__ int64_t survival(int R, int gamma, int gs, bool keys, int32_t *err, SchedShared &sh) {
  bool bad = false;
  int64_t wsum = 0;
  for (int rho = threadIdx.x; rho < R; rho += kSchedThreads) {
    float run = 1.0f;
    float *row = sh.conf + rho * gs;
    for (int j = 1; j <= gamma; ++j) {
      float c = row[j - 1];
      if (!(c >= 0.0f && c <= 1.0f)) {
        bad = true;
        c = 0.0f;
      }
      c = c == 0.0f ? 0.0f : c;  // -0.0 is the probability 0: no sign in any product
      run = run * c;
      row[j - 1] = run;
      wsum += fixed_weight(run);
      if (keys) sh.keys[(j - 1) * R + rho] = cand_key(run, j, rho);
    }
  }
  if (bad) flag_error(err, kErrConfidence);
  return wsum;
}

// survival (sh.conf) -> a (global, [R][gamma]), coalesced
__device__ __forceinline__ void write_survival(float *a, int N, int gamma, int gs, SchedShared &sh) {
  for (int i = threadIdx.x; i < N; i += kSchedThreads) {
    const int rho = i / gamma;
    a[i] = sh.conf[rho * gs + (i - rho * gamma)];
  }
}

// ---- bitonic sort of P2 = 1024 E keys held in registers, E per thread in
//      blocked order (thread t holds positions t E .. t E + E - 1).  Strides
//      below E pair registers of one thread, strides below 64 E pair lanes of
//      one wave (lane distance s / E: DPP for 1, 2 and 8, ds_bpermute
//      otherwise), larger strides go through LDS.

// value of lane (lane ^ M) of a 32-bit register
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
  else {
    const int lane = (int)(threadIdx.x & (kWave - 1));
    return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ M) << 2, (int)v);
  }
}
// keep the smaller of (own, other) where keep_min, else the larger
__device__ __forceinline__ uint64_t keep_of(uint64_t x, uint64_t o, bool keep_min) {
  return ((x < o) != keep_min) ? o : x;
}
// one compare-exchange stage with lane ^ M
template <int E, int M>
__device__ __forceinline__ void lane_stage(uint64_t (&k)[E], bool keep_min) {
  uint64_t o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t lo = lane_xor<M>((uint32_t)k[e]), hi = lane_xor<M>((uint32_t)(k[e] >> 32));
    o[e] = ((uint64_t)hi << 32) | lo;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) k[e] = keep_of(k[e], o[e], keep_min);
}
// compare-exchange of register pairs (e, e + S), ascending where bit `size`
// of the position is clear
template <int E, int S>
__device__ __forceinline__ void reg_stage(uint64_t (&k)[E], int base, int size) {
  if constexpr (S < E) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & S) == 0) {
        const bool up = ((base + e) & size) == 0;
        const uint64_t x = k[e], y = k[e + S];
        const bool sw = (x > y) == up;
        k[e] = sw ? y : x;
        k[e + S] = sw ? x : y;
      }
  }
}
// Strides across waves: position p = e + E (lane + 64 wave) in the blocked
// layout.  For the levels that have such strides the keys are transposed
// through LDS into a layout where the wave bits of p are lane bits (lane =
// l0 + 4 wave_p, wave = l_hi, with l0 and l_hi the low two and high four lane
// bits of p), the cross-wave strides run as lane shuffles, and the keys go
// back for the rest of the level: two barriers per level (alternating LDS
// buffers) instead of two per stride.
template <int E>
__device__ __forceinline__ int transposed_base() {
  constexpr int LE = E == 1 ? 0 : E == 2 ? 1 : E == 4 ? 2 : 3;
  const int lane = (int)(threadIdx.x & (kWave - 1)), wave = (int)threadIdx.x / kWave;
  return ((lane & 3) << LE) | (wave << (LE + 2)) | ((lane >> 2) << (LE + 6));
}
// LDS word of key position p in an exchange.  The low five bits of the word
// (its bank pair) take, besides the lane bits each layout already has there,
// the lane bits it lacks: the blocked layout's bits 5 .. 4 + log2(E) go to
// the register bits 0 .. log2(E) - 1, the transposed layout's lane bits at
// log2(E) + 6 .. go to the register bits and to the wave bits at
// log2(E) + 2 .. 4.  Each register e of the 32 lanes of a half wave then
// writes or reads 32 different bank pairs in both layouts (without it 16
// lanes shared one at E = 8: the cross-wave levels of an 8192-key sort took
// ~11 µs each).  A bijection on [0, 1024 E): only bits 0 .. 4 change, by a
// function of bits 5 and up.
template <int E>
__device__ __forceinline__ int exchange_word(int p) {
  constexpr int LE = E == 1 ? 0 : E == 2 ? 1 : E == 4 ? 2 : 3;
  const int lo = ((p >> 5) ^ (p >> (LE + 6))) & (E - 1);
  const int hi = ((p >> (2 * LE + 6)) & ((1 << (3 - LE)) - 1)) << (LE + 2);
  return p ^ lo ^ hi;
}
template <int E>
__device__ __forceinline__ void exchange(uint64_t (&k)[E], uint64_t *buf, int from, int to) {
#pragma unroll
  for (int e = 0; e < E; ++e) buf[exchange_word<E>(from + e)] = k[e];
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) k[e] = buf[exchange_word<E>(to + e)];
}
template <int E>
__device__ __forceinline__ void local_stage(uint64_t (&k)[E], int base, int size, int s) {
  const bool keep_min = ((base & s) == 0) == ((base & size) == 0);
  if (s >= E) {
    switch (s / E) {
      case 1: lane_stage<E, 1>(k, keep_min); break;
      case 2: lane_stage<E, 2>(k, keep_min); break;
      case 4: lane_stage<E, 4>(k, keep_min); break;
      case 8: lane_stage<E, 8>(k, keep_min); break;
      case 16: lane_stage<E, 16>(k, keep_min); break;
      default: lane_stage<E, 32>(k, keep_min); break;
    }
  } else if (s == 4) {
    reg_stage<E, 4>(k, base, size);
  } else if (s == 2) {
    reg_stage<E, 2>(k, base, size);
  } else {
    reg_stage<E, 1>(k, base, size);
  }
}
// The whole network is unrolled (P2 is a constant): no branches or loop
// control per stage, which would otherwise queue all 16 waves on the scalar
// unit.  buf0 and buf1 hold P2 keys each.
template <int E>
__device__ __forceinline__ void sort_keys(uint64_t (&k)[E], uint64_t *buf0, uint64_t *buf1) {
  constexpr int P2 = kSchedThreads * E, kCross = kWave * E;
  const int base = (int)threadIdx.x * E, tbase = transposed_base<E>();
#pragma unroll
  for (int size = 2; size <= P2; size <<= 1) {
    if (size > kCross) {
      exchange<E>(k, buf0, base, tbase);
#pragma unroll
      for (int s = size >> 1; s >= kCross; s >>= 1) {
        const bool keep_min = ((tbase & s) == 0) == ((tbase & size) == 0);
        switch (s / kCross) {
          case 1: lane_stage<E, 4>(k, keep_min); break;
          case 2: lane_stage<E, 8>(k, keep_min); break;
          case 4: lane_stage<E, 16>(k, keep_min); break;
          default: lane_stage<E, 32>(k, keep_min); break;
        }
      }
      exchange<E>(k, buf1, tbase, base);
    }
#pragma unroll
    for (int s = (size > kCross ? kCross : size) >> 1; s > 0; s >>= 1) local_stage<E>(k, base, size, s);
  }
}

// One pass of the scheduler over the confidences c: survival, candidate
// keys, sort, fixed-point path, then by mode:
//   kPathEarly: n* = first n whose theta does not grow, theta_{n*}
//   kPathFull:  n* = smallest argmax of theta over n = 0..N, theta_{n*}
//   kPathTop:   n* given, theta_{n*}
// Returns n*; the admitted candidates (sorted positions < n*) stay in k.
enum { kPathEarly = 1, kPathFull = 2, kPathTop = 3 };
template <int E>
__device__ __forceinline__ int scheduler_pass(const ScheduleLaunch L, const float *c, float *a_out, int how,
                              int n_top, const double (&sps)[E + 1], uint64_t (&k)[E],
                              double *theta_out, SchedShared &sh) {
  const int R = L.R, gamma = L.gamma, N = R * gamma, gs = gamma | 1;
  const int base = (int)threadIdx.x * E;
  stage_confidences(c, N, gamma, gs, sh);
  survival(R, gamma, gs, true, L.err, sh);
  __syncthreads();
  if (a_out) write_survival(a_out, N, gamma, gs, sh);
#pragma unroll
  for (int e = 0; e < E; ++e) k[e] = base + e < N ? sh.keys[base + e] : ~(uint64_t)0;
  sort_keys<E>(k, sh.keys, sh.keys2);

  // fixed-point path: A_i = sum of the weights before sorted position i
  int64_t wgt[E], lsum = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    wgt[e] = base + e < N ? fixed_weight(key_a(k[e])) : 0;
    lsum += wgt[e];
  }
  int64_t total;
  const int64_t excl = sched_exclusive_scan_i64(lsum, sh, &total);
  const double inv32 = 1.0 / 4294967296.0;
  int n_star = n_top;
  if (how == kPathEarly) {  // first n with !(theta_{n+1} > theta_n)
    int cand = 0x7fffffff;
    int64_t A = excl;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + e;
      if (i < N) {
        const double prev = ((double)R + (double)A * inv32) * sps[e];  // theta_i
        A += wgt[e];
        const double th = ((double)R + (double)A * inv32) * sps[e + 1];  // theta_{i+1}
        if (cand == 0x7fffffff && !(th > prev)) cand = i;
      }
    }
    n_star = sched_min_int(cand, sh);
    if (n_star == 0x7fffffff) n_star = N;
  } else if (how == kPathFull) {  // smallest argmax over n = 0..N
    double best = -INFINITY;
    int best_n = 0x7fffffff;
    int64_t A = excl;
    if (threadIdx.x == 0) {
      best = ((double)R + 0.0 * inv32) * sps[0];  // theta_0 = R SPS[R]
      best_n = 0;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = base + e;
      if (i < N) {
        A += wgt[e];
        const double th = ((double)R + (double)A * inv32) * sps[e + 1];
        if (th > best) {
          best = th;
          best_n = i + 1;
        }
      }
    }
    sched_argmax(&best, &best_n, sh);
    n_star = best_n;
  }
  // theta_{n*}: the thread holding sorted position n* - 1 (thread 0 for n* = 0)
  if (n_star == 0) {
    if (threadIdx.x == 0) *theta_out = ((double)R + 0.0 * inv32) * sps[0];
  } else if (base < n_star && n_star <= base + E) {
    // running values, no register array indexed by n* - base
    int64_t A = excl;
    double th = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      A += wgt[e];
      const double t = ((double)R + (double)A * inv32) * sps[e + 1];
      th = base + e + 1 == n_star ? t : th;
    }
    *theta_out = th;
  }
  return n_star;
}

// SPS[R + base + e] for e = 0..E (positions this thread's path values use)
template <int E>
__device__ __forceinline__ void prefetch_sps(const ScheduleLaunch L, double (&sps)[E + 1]) {
  const int N = L.R * L.gamma, base = (int)threadIdx.x * E;
#pragma unroll
  for (int e = 0; e <= E; ++e) sps[e] = base + e <= N ? L.SPS[L.R + base + e] : 0.0;
}

// THRESHOLD mode: survival in place (as for the sort) and, per request, the
// number of leading positions with c >= threshold and the fixed-point weight
// of those positions; returns the thread's weight sum, lengths in len[].
constexpr int kMaxReqPerThread = kMaxCandidates / kSchedThreads;
__device__ __forceinline__ int64_t threshold_survival(int R, int gamma, int gs, float thr,
                                                      int32_t *err, SchedShared &sh,
                                                      int (&len)[kMaxReqPerThread]) {
  bool bad = false;
  int64_t wsum = 0;
#pragma unroll
  for (int q = 0; q < kMaxReqPerThread; ++q) {
    len[q] = 0;
    const int rho = (int)threadIdx.x + q * kSchedThreads;
    if (rho >= R) continue;
    float run = 1.0f;
    float *row = sh.conf + rho * gs;
    bool kept = true;
    for (int j = 1; j <= gamma; ++j) {
      float c = row[j - 1];
      if (!(c >= 0.0f && c <= 1.0f)) {
        bad = true;
        c = 0.0f;
      }
      c = c == 0.0f ? 0.0f : c;  // -0.0 -> +0.0, as in the ranked modes
      run = run * c;
      row[j - 1] = run;
      kept = kept && c >= thr;
      if (kept) {
        len[q] = j;
        wsum += fixed_weight(run);
      }
    }
  }
  if (bad) flag_error(err, kErrConfidence);
  return wsum;
}

template <int E>
__device__ __forceinline__ void schedule_body(const ScheduleLaunch L, SchedShared &sh, double *s_theta) {
  const int R = L.R, gamma = L.gamma, N = R * gamma;
  int n_star = N;
  double theta = NAN;
  uint64_t k[E];
  int len[kMaxReqPerThread];  // THRESHOLD mode: kept lengths of requests tid + q 1024
  if (L.mode == 4) {
    const int gs = gamma | 1;
    stage_confidences(L.c, N, gamma, gs, sh);
    const int64_t wsum = threshold_survival(R, gamma, gs, L.threshold, L.err, sh, len);
    __syncthreads();
    if (L.a) write_survival(L.a, N, gamma, gs, sh);
    int64_t nl = 0;
#pragma unroll
    for (int q = 0; q < kMaxReqPerThread; ++q) nl += len[q];
    int64_t A, n_total;
    sched_exclusive_scan_i64(wsum, sh, &A);
    sched_exclusive_scan_i64(nl, sh, &n_total);
    n_star = (int)n_total;
    if (threadIdx.x == 0 && L.SPS != nullptr)
      theta = ((double)R + (double)A * (1.0 / 4294967296.0)) * L.SPS[R + n_star];
  } else if (L.mode == 0) {
    if (L.c != nullptr) {
      const int gs = gamma | 1;
      stage_confidences(L.c, N, gamma, gs, sh);
      const int64_t local = survival(R, gamma, gs, false, L.err, sh);
      __syncthreads();
      if (L.a) write_survival(L.a, N, gamma, gs, sh);
      int64_t total;
      sched_exclusive_scan_i64(local, sh, &total);
      if (threadIdx.x == 0 && L.SPS != nullptr)
        theta = ((double)R + (double)total * (1.0 / 4294967296.0)) * L.SPS[R + N];
    }
  } else {
    double sps[E + 1];
    prefetch_sps<E>(L, sps);
    if (L.mode == 3) {  // capacity from round t-2: full search on its own path
      double unused = 0.0;
      n_star = scheduler_pass<E>(L, L.c_prev2, nullptr, kPathFull, 0, sps, k, &unused, sh);
      __syncthreads();
      n_star = scheduler_pass<E>(L, L.c, L.a, kPathTop, n_star, sps, k, &theta, sh);
    } else {
      n_star = scheduler_pass<E>(L, L.c, L.a, L.mode, 0, sps, k, &theta, sh);
    }
  }
  __syncthreads();  // done with sh.conf: it becomes sh.ell
  if (!isnan(theta)) *s_theta = theta;  // exactly one thread holds it
  if (L.mode == 4) {
#pragma unroll
    for (int q = 0; q < kMaxReqPerThread; ++q) {
      const int rho = (int)threadIdx.x + q * kSchedThreads;
      if (rho < R) sh.ell[rho] = len[q];
    }
  } else {
    for (int rho = threadIdx.x; rho < R; rho += kSchedThreads) sh.ell[rho] = L.mode == 0 ? gamma : 0;
  }
  __syncthreads();
  if (L.mode != 0 && L.mode != 4) {
    // admitted candidates are a prefix of each request (keys increase with
    // depth along a request): its admitted count is its deepest admitted j
    const int base = (int)threadIdx.x * E;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (base + e < n_star) atomicMax(&sh.ell[key_rho(k[e])], key_j(k[e]));
    __syncthreads();
  }
  // row offsets: exclusive scan of 1 + ell in request order
  constexpr int kMaxPerThread = kMaxCandidates / kSchedThreads;  // R <= N <= 8192
  const int cpr = (R + kSchedThreads - 1) / kSchedThreads;
  const int r0 = min((int)threadIdx.x * cpr, R), r1 = min(r0 + cpr, R);
  int lens[kMaxPerThread];
  int64_t local = 0;
#pragma unroll
  for (int q = 0; q < kMaxPerThread; ++q) {
    const int rho = r0 + q;
    lens[q] = rho < r1 ? sh.ell[rho] : 0;
    if (rho < r1) {
      L.ell[rho] = lens[q];
      local += 1 + lens[q];
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
    *L.n_admitted = L.mode == 0 ? N : n_star;
  }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleLaunch L) {
  __shared__ SchedShared sh;
  __shared__ double s_theta;
  if (threadIdx.x == 0) s_theta = NAN;
  __syncthreads();
  // keys per thread: the sort pads N to 1024 E
  const int N = L.R * L.gamma;
  if (N <= kSchedThreads) schedule_body<1>(L, sh, &s_theta);
  else if (N <= 2 * kSchedThreads) schedule_body<2>(L, sh, &s_theta);
  else if (N <= 4 * kSchedThreads) schedule_body<4>(L, sh, &s_theta);
  else schedule_body<8>(L, sh, &s_theta);
  __syncthreads();
  if (threadIdx.x == 0) *L.theta = s_theta;
}

hipError_t launch_schedule(const ScheduleLaunch &L, hipStream_t stream) {
  DSPARK_LAUNCH("schedule", stream, schedule_kernel, 1, kSchedThreads, L);
  return hipGetLastError();
}

}  // namespace dspark
