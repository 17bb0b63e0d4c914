// Inverse-CDF draw of one drafted token (Bangkok 4.1, left-to-right
// sampling; Blog "Markov sequential head"), shared by the per-step sampling
// kernel and the persistent draft kernel.
//
// Sampling is an inverse CDF in two levels.  The workgroup of request rho
// rescales the row's tile partials (m_t, s_t) to the row maximum, scans them
// to find the tile whose cumulative mass first exceeds u * S, recomputes z for
// that tile alone (bit-identical to the product kernels: same matrix-core
// instruction sequence and operand order), and scans inside the tile.  Only
// the 128-column tile is re-read, never the row.
#pragma once
#include "bias_tile.h"

namespace dspark {

struct SampleParams {
  int R, gamma, V, r, n_tiles, k;
  float invT;
  const void *U, *W1, *W2;
  const void *A_cur;         // [R][r]: W1[x_{k-1}] of every request
  const int32_t *a_tokens;   // or, if set, x_{k-1} (A_cur row rho = W1[a_tokens[rho]])
  void *A_next;              // [R][r]: receives W1[x_k] (NULL at the last step)
                             // (k and A_next are passed to sample_row separately)
  int32_t *x;
  float *q_stats, *q_x;
  const float2 *tile_stats;  // [R][n_tiles]
  uint64_t seed, round;
  // confidence head (Bangkok 4.2.1): c_k = sigmoid((sh[rho][k] + w_e . W1[x_{k-1}] + b) / T_k)
  // with sequential temperature scaling's T_k (Blog "Sequential temperature scaling")
  const float *sh;           // [R][gamma] = w_h . h_k, or NULL
  const float *w_e;          // [r] (the last r weights of w_conf)
  float b_conf;
  const float *conf_temp;    // [gamma] T_k, or NULL (1)
  float *c;
  // teacher forcing: if set, x_k is the label x_force[rho][k-1] instead of a
  // draw, and logq_x (if set) receives log q_k(x_k)
  const int32_t *x_force;
  float *logq_x;
  int32_t *err;
};

// LDS of one draw (the caller's; reused row after row with a barrier between)
struct SampleLds {
  float zbuf[kTileN];
  float red_max[4], red_sum[4];
  int red_found[4], red_last[4];
  float s_before, s_mt, s_u;
};

// The persistent draft's side of a draw (sample_row<T, true>), where other
// workgroups of the same kernel write the row's tile partials and read the
// draw: the partial words are polled in place until none reads kTileEmpty,
// then reset to kTileEmpty (the writers of the step two later find them so),
// and the draw is published as (k << 32) | x_k.  All these accesses are
// device-coherent.
struct PersistIo {
  uint64_t *tiles;  // the step's [R][n_tiles] partial words (bits of float2 (max z, sum))
  uint64_t *pub;    // [R]
  int *abort;       // the workgroup's LDS word, set when a wait runs out
};
constexpr uint64_t kTileEmpty = ~0ull;  // a NaN pattern (writers store another for it)
constexpr int kSpinLimit = 1 << 18;     // polls before a wait gives up

// Draw x_k of request rho (k = position, 1-based; p.k is not read); called by
// all kBlock threads of the workgroup.  arow: W1[x_{k-1}] of rho in LDS (r
// elements, 16-byte aligned).  With stage_arow the function first copies that
// row there itself (from A_cur, or from W1[a_tokens[rho]] in place);
// otherwise the caller has put it there.  A_next (or NULL) receives W1[x_k].
// Without kPersist the tile partials (p.tile_stats), and the transition rows
// read through A_cur or a_tokens, must be visible before the call; with it
// see PersistIo.  KS > 0: r = 16 KS (bf16), fixed at compile time.
// kFreshTid: the thread index is made opaque to the compiler at each call,
// so that no address derived from it is held across a caller's loop (held
// ones went to scratch, and a reload waits for every load in flight).
// Returns false, in every thread, only when a persistent wait ran out
// (kErrSync).
template <typename T, bool kPersist = false, int KS = 0, bool kFreshTid = false>
__device__ __forceinline__ bool sample_row(const SampleParams &p, int k, void *A_next, int rho,
                                           T *arow, bool stage_arow, SampleLds &sl,
                                           const PersistIo &io = PersistIo{}) {
  constexpr int kCpt = kMaxTiles / kBlock;  // tiles per thread, at most
  float *zbuf = sl.zbuf;
  float *red_max = sl.red_max, *red_sum = sl.red_sum;
  int *red_found = sl.red_found, *red_last = sl.red_last;
  float &s_before = sl.s_before, &s_mt = sl.s_mt, &s_u = sl.s_u;

  int tid_raw = threadIdx.x;
  if constexpr (kFreshTid) asm volatile("" : "+v"(tid_raw));
  const int tid = tid_raw, lane = tid & (kWave - 1);
  const int wave = kFreshTid ? __builtin_amdgcn_readfirstlane(tid / kWave) : tid / kWave;
  const int V = p.V, r = p.r, nT = p.n_tiles;
  const int64_t slot = (int64_t)rho * p.gamma + (k - 1);
  constexpr int kPer = 16 / (int)sizeof(T);
  const int pieces = r * (int)sizeof(T) / 16;

  // 1. W1[x_{k-1}] (= A_k[rho]) to LDS; this thread's contiguous tiles
  //    [t0, t1) of the row's partials into registers, one round trip
  const int cpt = (nT + kBlock - 1) / kBlock;
  const int t0 = min(tid * cpt, nT), t1 = min(t0 + cpt, nT);
  float2 pt[kCpt];
  const int forced_raw = p.x_force != nullptr ? p.x_force[slot] : 0;
  {
    const T *Acur = reinterpret_cast<const T *>(p.A_cur) + (int64_t)rho * r;
    if (p.a_tokens != nullptr)  // validated (and flagged) by the product kernel
      Acur = reinterpret_cast<const T *>(p.W1) + (int64_t)min(max(p.a_tokens[rho], 0), V - 1) * r;
    uint4 a = make_uint4(0, 0, 0, 0);
    if (stage_arow && tid < pieces) a = *reinterpret_cast<const uint4 *>(Acur + tid * kPer);
    if constexpr (kPersist) {
      // poll the words not yet written (all in flight at once), then reset them
      uint64_t *ts = io.tiles + (int64_t)rho * nT;
      uint64_t v[kCpt];
      unsigned missing = 0;
#pragma unroll
      for (int j = 0; j < kCpt; ++j)
        if (t0 + j < t1) missing |= 1u << j;
      for (int spins = 0; missing != 0u; ++spins) {
        if (spins > kSpinLimit) {
          *io.abort = 1;
          flag_error(p.err, kErrSync);
          break;
        }
        if (spins > 0) __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < kCpt; ++j)
          if (missing & (1u << j)) v[j] = ld_coherent(ts + t0 + j);
#pragma unroll
        for (int j = 0; j < kCpt; ++j)
          if ((missing & (1u << j)) && v[j] != kTileEmpty) missing &= ~(1u << j);
      }
#pragma unroll
      for (int j = 0; j < kCpt; ++j) {
        pt[j] = t0 + j < t1 ? __builtin_bit_cast(float2, v[j]) : make_float2(-INFINITY, 0.0f);
        if (t0 + j < t1) st_coherent(ts + t0 + j, kTileEmpty);
      }
    } else {
      const float2 *ts = p.tile_stats + (int64_t)rho * nT;
#pragma unroll
      for (int j = 0; j < kCpt; ++j) pt[j] = t0 + j < t1 ? ts[t0 + j] : make_float2(-INFINITY, 0.0f);
    }
    // the draw's uniform (a scalar Philox chain) is formed while the loads
    // are in flight: the LDS store keeps it ahead of the first barrier
    if (tid == 0) s_u = uniform01(p.seed, p.round, (uint64_t)k, (uint64_t)rho, kStreamDraft);
    if (stage_arow && tid < pieces) *reinterpret_cast<uint4 *>(arow + tid * kPer) = a;
  }
  // 2. row maximum, then tile masses w_t = s_t exp(m_t - m) and their
  //    exclusive scan in tile order (one barrier each)
  float lm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kCpt; ++j) lm = fmaxf(lm, pt[j].x);
  lm = wave_max(lm);
  if (lane == 0) red_max[wave] = lm;
  __syncthreads();
  if (kPersist && *io.abort != 0) return false;
  const float m = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
  float w[kCpt];
  float ls = 0.0f;
#pragma unroll
  for (int j = 0; j < kCpt; ++j) {
    w[j] = t0 + j < t1 ? pt[j].y * fexp(pt[j].x - m) : 0.0f;
    ls += w[j];
  }
  const float inc = wave_inclusive_scan(ls);
  if (lane == kWave - 1) red_sum[wave] = inc;
  __syncthreads();
  float before_wave = 0.0f;
  for (int i = 0; i < wave; ++i) before_wave += red_sum[i];
  const float S = ((red_sum[0] + red_sum[1]) + red_sum[2]) + red_sum[3];
  const float base = before_wave + (inc - ls);
  const bool finite = isfinite(m) && isfinite(S) && S > 0.0f;

  // 3. the tile holding the draw: the first tile whose cumulative mass
  //    exceeds u * S (else, rounding having left no crossing, the last tile
  //    with mass)
  const float u = s_u;
  const float target = u * S;
  int found = 0x7fffffff, lastpos = -1;
  {
    float run = base;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      const float nx = run + w[j];
      if (found == 0x7fffffff && target < nx && w[j] > 0.0f) found = t0 + j;
      if (w[j] > 0.0f) lastpos = t0 + j;
      run = nx;
    }
  }
  found = wave_min_int(found);
  lastpos = wave_max_int(lastpos);
  if (lane == 0) { red_found[wave] = found; red_last[wave] = lastpos; }
  __syncthreads();
  int tstar = min(min(red_found[0], red_found[1]), min(red_found[2], red_found[3]));
  if (tstar == 0x7fffffff) tstar = max(max(red_last[0], red_last[1]), max(red_last[2], red_last[3]));
  if (tstar < 0 || !finite) {
    if (tid == 0) flag_error(p.err, kErrNonFinite);
    tstar = 0;
  }
  int forced = -1;  // the label's column, under teacher forcing
  if (p.x_force != nullptr) {
    forced = forced_raw;
    if (forced < 0 || forced >= V) {
      if (tid == 0) flag_error(p.err, kErrToken);
      forced = 0;
    }
    tstar = forced / kTileN;
  }
  if (t0 <= tstar && tstar < t1) {  // the owner of the tile: mass before it, its max
    float run = base;
    float mt = 0.0f;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
      if (t0 + j < tstar) run += w[j];
      if (t0 + j == tstar) mt = pt[j].x;
    }
    s_before = run;  // read after the barrier that follows the recompute
    s_mt = mt;
  }

  // 4. recompute z of that tile, bit-identical to the fused kernel
  const T *Urow = reinterpret_cast<const T *>(p.U) + slot * V;
  recompute_tile_v<T, true, KS>(arow, reinterpret_cast<const T *>(p.W2), Urow, V, r, tstar,
                                rho & 31, zbuf);
  // persistent: every wave's partial resets have completed before the draw is
  // published (the step two later writes those words again)
  if (kPersist) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 5. scan inside the tile (wave 0, two columns per lane, left to right);
  //    z = (acc + u) / T, the draft's exact arithmetic
  if (wave == 0) {
    const float mt = s_mt;
    const float scale = fexp(mt - m);
    const float z0 = zbuf[2 * lane] * p.invT, z1 = zbuf[2 * lane + 1] * p.invT;
    const float e0 = fexp(z0 - mt), e1 = fexp(z1 - mt);
    const float incl = wave_inclusive_scan(e0 + e1);
    const float exc = wave_prev_lane(incl);
    const float cdf0 = s_before + scale * (exc + e0);
    const float cdf1 = s_before + scale * ((exc + e0) + e1);
    int pick = 0x7fffffff;
    if (target < cdf0 && e0 > 0.0f) pick = 2 * lane;
    else if (target < cdf1 && e1 > 0.0f) pick = 2 * lane + 1;
    pick = wave_min_int(pick);
    if (forced >= 0) {
      pick = forced - tstar * kTileN;
    } else if (pick == 0x7fffffff) {
      int lp = -1;
      if (e0 > 0.0f) lp = 2 * lane;
      if (e1 > 0.0f) lp = 2 * lane + 1;
      pick = wave_max_int(lp);
      if (pick < 0) pick = 0;
    }
    const float zp = __shfl(pick & 1 ? z1 : z0, pick >> 1);
    const int xk = tstar * kTileN + pick;  // in [0, V): a picked column has positive mass
    if (kPersist && lane == 0)  // first: the other workgroups wait for it
      st_coherent(io.pub + rho, ((uint64_t)k << 32) | (uint32_t)min(max(xk, 0), V - 1));
    if (lane == 0) {
      p.x[slot] = finite ? xk : -1;
      p.q_stats[2 * slot] = m;
      p.q_stats[2 * slot + 1] = S;
      p.q_x[slot] = fexp(zp - m) / S;
      if (p.logq_x != nullptr) p.logq_x[slot] = (zp - m) - logf(S);
    }
    // 7. the next step's transition row A_{k+1}[rho] = W1[x_k], by this wave
    //    (no barrier: the token is in its registers)
    if (A_next != nullptr && lane < pieces) {
      const int xc = min(max(xk, 0), V - 1);
      T *dst = reinterpret_cast<T *>(A_next) + (int64_t)rho * r + lane * kPer;
      const uint4 w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const T *>(p.W1) +
                                                       (int64_t)xc * r + lane * kPer);
      *reinterpret_cast<uint4 *>(dst) = w;
    }

  }

  // 6. confidence head on [h_k ; W1[x_{k-1}]], at the position's temperature (wave 1)
  if (p.sh != nullptr && wave == 1) {
    float tk = p.conf_temp != nullptr ? p.conf_temp[k - 1] : 1.0f;  // in flight with the dot
    float acc = 0.0f;
    for (int i = lane; i < r; i += kWave) acc = fmaf(p.w_e[i], Elem<T>::at(arow, i), acc);
    acc = wave_sum(acc);
    if (lane == 0) {
      if (!(tk > 0.0f) || !isfinite(tk)) {
        flag_error(p.err, kErrConfidence);
        tk = 1.0f;
      }
      const float s = p.sh[slot] + acc + p.b_conf;
      p.c[slot] = 1.0f / (1.0f + expf(-s / tk));
    }
  }
  return true;
}

}  // namespace dspark
