// Exact speculative-sampling verification of the flattened ragged batch
// (Blog, "One-token exactness", "Why only the longest accepted prefix
// survives", "Variable-length verification without wasting kernels"; KB
// sections 7-8).  The launches:
//
//  1. row_chunk_stats_kernel: one HBM pass over the sum(1 + ell) target rows,
//     (max, sum exp) per quarter row; the last row of every request (its bonus
//     position) also keeps per-tile partials for sampling.
//  2. the product: recompute z_k of every verified draft with the draft's
//     arithmetic, stream U_k and P_k once, emit per-tile
//     (sum min(p, q), sum (p - q)_+) -- verify_stationary_kernel (W2 held on
//     chip, after verify_row_stats_kernel; verify_stationary.hip) or
//     stream_tile_kernel<verify> (bias_tile.h).
//  3. verify_finalize_kernel: per request, one workgroup for the accept tests
//     in order, the first rejection and the residual or bonus draw by a
//     two-level inverse CDF, and one for c*_k.
#include "bias_tile.h"
#include "kernels.h"
#include "trace.h"

namespace dspark {

struct RowStatsParams {
  int n_rows, V, n_tiles;
  float invT;
  const void *X;              // [n_rows][V]
  const int32_t *row_offset;  // verify: rows >= row_offset[R] are unused; else NULL
  int R;
  float2 *chunks;             // [n_rows][kChunks]
  float2 *bonus_tiles;        // [R][n_tiles], verify only
  int32_t *err;
  // verify only: the compact-row map of the verified drafts
  int gamma;
  const int32_t *x0, *x;
  int4 *row_map;              // [R*gamma]: (rho, k, x_{k-1}, target row)
  int r;
  const void *W1;
  void *A_rows;               // [R*gamma][r]: W1[x_{k-1}] of compact row i
  const void *A_given;        // or, if set, row ((k-1) R + rho) of [gamma][R][r]
};

// One quarter of one row per workgroup, in rounds of kBatch 16-byte pieces per
// thread (all in flight together; few registers, so many workgroups share a
// compute unit).  The request lookup of the row runs while the first round's
// loads are outstanding.  Per round:
//   - a verified-draft row: max and sum of exp over the thread's elements in
//     two passes, then one workgroup reduction;
//   - the last row of a request (its bonus position): (max, sum of exp) per
//     128-column tile as well, kept for the bonus draw.
// exp(x / T - m) is formed as 2^((x - x_max) log2(e) / T), with m = x_max / T
// exactly (T > 0): x - x_max is exact near the maximum, where the mass is (a
// single fused multiply-add with x_max log2(e) / T rounded was 4% faster but
// shifts every term by up to half an ulp of that product).
template <typename T>
__global__ __launch_bounds__(kBlock) void row_chunk_stats_kernel(RowStatsParams p) {
  __shared__ float red[8];
  constexpr int kPer = Elem<T>::kPerVec;
  constexpr int kBatch = 2;                  // pieces per thread per round (4: 48.9 us, 6: 51.7)
  constexpr int kG = kTileN / kPer;          // threads per tile (bf16: 16, fp32: 32)
  const int c = blockIdx.x, tid = threadIdx.x;
  const int V = p.V, nT = p.n_tiles;
  int used = p.n_rows;
  if (p.row_offset != nullptr) {
    used = p.row_offset[p.R];
    if (used > p.n_rows) {
      if (blockIdx.y == 0 && c == 0 && tid == 0) flag_error(p.err, kErrLength);
      used = p.n_rows;
    }
  }
  // rows blockIdx.y, blockIdx.y + gridDim.y, ... below the rows in use (the
  // host sizes the grid by its bound on them, capped; see the launch)
  for (int row = blockIdx.y; row < used; row += gridDim.y) {
  const int tpc = (nT + kChunks - 1) / kChunks;
  const int tb = min(c * tpc, nT), te = min(tb + tpc, nT);
  // an empty chunk (c tpc >= nT) starts at V, so that its clamped loads read
  // the row's last piece and never the bytes past it
  const int vb = min(tb * kTileN, V), ve = min(te * kTileN, V);
  const int npc = (ve - vb + kPer - 1) / kPer;  // pieces in the chunk (V % kPer == 0)
  const T *X = reinterpret_cast<const T *>(p.X) + (int64_t)row * V + vb;
  const float cl = p.invT * kLog2e;

  float M = -INFINITY, S = 0.0f;  // running (max of x, sum of 2^((x - M) cl))
  int rho = -1;                   // set for the last row of a request
  // rounds of kBatch pieces per thread, double-buffered: the loads of round
  // i + 1 are in flight while round i is reduced (past the chunk they read
  // its last piece again, and the results are not used)
  constexpr int kRound = kBatch * kBlock;
  auto issue = [&](u32x4 (&raw)[kBatch], int p0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      raw[j] = ld_stream4(X + (int64_t)min(p0 + j * kBlock + tid, npc - 1) * kPer);
  };
  u32x4 cur[kBatch], nxt[kBatch];
  issue(cur, 0);
  issue(nxt, kRound);
  if (p.row_offset != nullptr) {
    // request of the row: the last rho with row_offset[rho] <= row, as the
    // number of rho in [1, R) with row_offset[rho] <= row (the offsets are
    // nondecreasing), counted by every wave with ballots over loads that are
    // all in flight at once (a binary search took one round trip per step)
    const int lane = tid & (kWave - 1);
    int lo = 0;
    for (int t0 = 1; t0 < p.R; t0 += 4 * kWave) {
      int v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u * kWave + lane;
        const int o = p.row_offset[min(t, p.R)];
        v[u] = t < p.R ? o : INT_MAX;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) lo += __popcll(__ballot(v[u] <= row));
    }
    const int base = p.row_offset[lo];
    if (p.row_offset[lo + 1] - 1 == row) {
      rho = lo;  // the bonus position keeps tile partials
    } else if (c == 0 && tid < 32) {
      // a verified draft (k <= ell): its entry of the compact-row map and
      // its transition row W1[x_{k-1}] for the verify pass
      const int k = row - base + 1, i = row - lo;
      if (k >= 1 && k <= p.gamma && i >= 0 && i < p.R * p.gamma) {
        int prev = k == 1 ? p.x0[lo] : p.x[(int64_t)lo * p.gamma + k - 2];
        if (prev < 0 || prev >= V) {
          if (tid == 0) flag_error(p.err, kErrToken);
          prev = prev < 0 ? 0 : V - 1;
        }
        if (tid == 0) p.row_map[i] = make_int4(lo, k, prev, row);
        constexpr int kPerA = 16 / (int)sizeof(T);
        if (tid < p.r * (int)sizeof(T) / 16)
          *reinterpret_cast<uint4 *>(reinterpret_cast<T *>(p.A_rows) + (int64_t)i * p.r +
                                     tid * kPerA) =
              *reinterpret_cast<const uint4 *>(
                  (p.A_given != nullptr
                       ? reinterpret_cast<const T *>(p.A_given) + ((int64_t)(k - 1) * p.R + lo) * p.r
                       : reinterpret_cast<const T *>(p.W1) + (int64_t)prev * p.r) +
                  tid * kPerA);
      } else if (tid == 0) {
        flag_error(p.err, kErrLength);
      }
    }
  }
  auto reduce = [&](const u32x4 (&raw)[kBatch], int p0) __attribute__((always_inline)) {
    if (rho < 0) {
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float x[kPer];
        unpack16(raw[j], (T *)nullptr, x);
        const bool in = p0 + j * kBlock + tid < npc;
#pragma unroll
        for (int q = 0; q < kPer; ++q) bm = fmaxf(bm, in ? x[q] : -INFINITY);
      }
      if (bm != -INFINITY) {
        const float mn = fmaxf(M, bm);
        float sb = 0.0f;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          float x[kPer];
          unpack16(raw[j], (T *)nullptr, x);
          const bool in = p0 + j * kBlock + tid < npc;
          float e = 0.0f;
#pragma unroll
          for (int q = 0; q < kPer; ++q) e += exp2_fast((x[q] - mn) * cl);
          sb += in ? e : 0.0f;
        }
        S = fmaf(S, exp2_fast((M - mn) * cl), sb);
        M = mn;
      }
    } else {
      // tile of piece (p0 + j kBlock + tid): kG consecutive threads share one
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int pc = p0 + j * kBlock + tid;
        const bool in = pc < npc;
        if (p0 + j * kBlock >= npc) continue;  // uniform: no piece of this round left
        float x[kPer];
        unpack16(raw[j], (T *)nullptr, x);
        float lm = -INFINITY;
#pragma unroll
        for (int q = 0; q < kPer; ++q) lm = fmaxf(lm, in ? x[q] : -INFINITY);
        const float mt = group_max<kG>(lm);
        float ls = 0.0f;
        if (in) {
#pragma unroll
          for (int q = 0; q < kPer; ++q) ls += exp2_fast((x[q] - mt) * cl);
        }
        const float st = group_sum<kG>(ls);
        const int t = tb + pc / kG;
        if (in && (tid % kG) == 0) {
          p.bonus_tiles[(int64_t)rho * nT + t] = make_float2(mt * p.invT, st);
          if (mt > M) {
            S = S * exp2_fast((M - mt) * cl) + st;
            M = mt;
          } else {
            S += st * exp2_fast((mt - M) * cl);
          }
        }
      }
    }
  };
  for (int p0 = 0; p0 < npc; p0 += 2 * kRound) {
    reduce(cur, p0);
    issue(cur, p0 + 2 * kRound);
    if (p0 + kRound < npc) reduce(nxt, p0 + kRound);
    issue(nxt, p0 + 3 * kRound);
  }
  // workgroup (max, sum): x-units, then m = x_max / T
  const float mx = block_max(M, red);
  const float sx = block_sum(M == -INFINITY ? 0.0f : S * exp2_fast((M - mx) * cl), red);
  if (tid == 0) {
    const float m = mx * p.invT;
    p.chunks[(int64_t)row * kChunks + c] = make_float2(m, sx);
    if (vb < ve && !(isfinite(m) && isfinite(sx))) flag_error(p.err, kErrNonFinite);
  }
  }
}

// ------------------------------------------------------------------ finalize
struct FinalizeParams {
  int R, gamma, V, r, n_tiles, rows_capacity;
  float invT;
  const int32_t *ell, *row_offset;
  const void *P, *U, *W1, *W2;
  const void *A_given;  // [gamma][R][r] transition rows, or NULL (W1[x_{k-1}])
  const int32_t *x0, *x;
  const float *q_stats, *q_x;
  uint64_t seed, round;
  const float2 *p_chunks, *bonus_tiles, *pair_partials;
  int32_t *n_acc, *y;
  float *c_star;
  int32_t *err;
};

// Two-level inverse CDF over tile masses already in wbuf[0..nT): returns the
// tile holding u * total and writes the mass before it to *before.
__device__ int pick_tile(const float *wbuf, int nT, float u, float *fred, int *ired,
                         float *s_before, float *total_out, float *target_out) {
  const int tid = threadIdx.x;
  const int cpt = (nT + kBlock - 1) / kBlock;
  const int t0 = min(tid * cpt, nT), t1 = min(t0 + cpt, nT);
  float ls = 0.0f;
  for (int t = t0; t < t1; ++t) ls += wbuf[t];
  float total;
  const float base = block_exclusive_scan(ls, fred, &total);
  const float target = u * total;
  int found = 0x7fffffff;
  float run = base;
  for (int t = t0; t < t1; ++t) {
    const float nx = run + wbuf[t];
    if (found == 0x7fffffff && target < nx && wbuf[t] > 0.0f) found = t;
    run = nx;
  }
  int tstar = block_min_int(found, ired);
  if (tstar == 0x7fffffff) {
    int lastpos = -1;
    for (int t = t0; t < t1; ++t)
      if (wbuf[t] > 0.0f) lastpos = t;
    tstar = block_max_int(lastpos, ired);
  }
  if (tstar < 0) tstar = 0;
  if (tid == 0) *s_before = 0.0f;
  __syncthreads();
  if (t0 <= tstar && tstar < t1) {
    float b = base;
    for (int t = t0; t < tstar; ++t) b += wbuf[t];
    *s_before = b;
  }
  __syncthreads();
  *total_out = total;
  *target_out = target;
  return tstar;
}

// In-tile scan of 128 masses ebuf[] (wave 0): first column whose cumulative
// mass before + scale * prefix exceeds target (positive mass only).
__device__ int pick_in_tile(const float *ebuf, float before, float scale, float target) {
  const int lane = threadIdx.x & (kWave - 1);
  const float e0 = ebuf[2 * lane], e1 = ebuf[2 * lane + 1];
  const float inc = wave_inclusive_scan(e0 + e1);
  const float exc = wave_prev_lane(inc);
  const float cdf0 = before + scale * (exc + e0);
  const float cdf1 = before + scale * ((exc + e0) + e1);
  int pick = 0x7fffffff;
  if (target < cdf0 && e0 > 0.0f) pick = 2 * lane;
  else if (target < cdf1 && e1 > 0.0f) pick = 2 * lane + 1;
  pick = wave_min_int(pick);
  if (pick == 0x7fffffff) {
    int lp = -1;
    if (e0 > 0.0f) lp = 2 * lane;
    if (e1 > 0.0f) lp = 2 * lane + 1;
    pick = wave_max_int(lp);
    if (pick < 0) pick = 0;
  }
  return pick;
}

// The request's slice of the ragged batch, checked against the batch bounds.
// An invalid slice runs as an empty one (every address stays in bounds).
struct RequestSlice {
  bool ok;
  int ell, base;
  int64_t d_off;  // compact index of (rho, k = 1)
};
__device__ __forceinline__ RequestSlice request_slice(const FinalizeParams &p, int rho, int ell_in,
                                                      int base_in, int next, int rows_used) {
  RequestSlice q;
  q.ok = ell_in >= 0 && ell_in <= p.gamma && base_in >= 0 && next == base_in + 1 + ell_in &&
         base_in + ell_in < p.rows_capacity && rows_used <= p.rows_capacity && base_in >= rho &&
         (int64_t)base_in - rho + ell_in <= (int64_t)p.R * p.gamma;
  q.ell = q.ok ? ell_in : 0;
  q.base = q.ok ? base_in : 0;
  q.d_off = q.ok ? (int64_t)q.base - rho : 0;
  return q;
}

// c*_k = sum over tiles of sum_v min(p, q) in tile order (NaN past ell), by a
// workgroup of its own: the accept tests and the final draw do not read it.
// Wave w takes k = w + 1, w + 5, ... two at a time, every tile load in flight
// (clamped past n_tiles, masked in the sum).
__device__ __forceinline__ void finalize_cstar(const FinalizeParams &p, int rho) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int gamma = p.gamma, nT = p.n_tiles;
  const RequestSlice q = request_slice(p, rho, p.ell[rho], p.row_offset[rho], p.row_offset[rho + 1],
                                       p.row_offset[p.R]);
  const int ell = q.ell;
  float *crow = p.c_star + (int64_t)rho * gamma;
  constexpr int kTpl = kMaxTiles / kWave;  // tiles per lane, at most
  for (int ka = 1 + wave; ka <= ell; ka += 2 * (kBlock / kWave)) {
    const int kb = ka + kBlock / kWave;
    const float2 *pa = p.pair_partials + (q.d_off + ka - 1) * nT;
    const float2 *pb = p.pair_partials + (q.d_off + min(kb, ell) - 1) * nT;
    float va[kTpl], vb[kTpl];
#pragma unroll
    for (int i = 0; i < kTpl; ++i) {
      const int t = min(lane + i * kWave, nT - 1);
      va[i] = pa[t].x;
      vb[i] = pb[t].x;
    }
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int i = 0; i < kTpl; ++i)
      if (lane + i * kWave < nT) {
        sa += va[i];
        sb += vb[i];
      }
    sa = wave_sum(sa);
    sb = wave_sum(sb);
    if (lane == 0) {
      crow[ka - 1] = sa;
      if (kb <= ell) crow[kb - 1] = sb;
    }
  }
  for (int k = ell + 1 + tid; k <= gamma; k += kBlock) crow[k - 1] = NAN;
}

// Workgroups [0, R): the accept tests, the first rejection and the final
// token of request rho = blockIdx.x; workgroups [R, 2R): c* of request
// blockIdx.x - R.
template <typename T>
__global__ __launch_bounds__(kBlock) void verify_finalize_kernel(FinalizeParams p) {
  if (blockIdx.x >= (unsigned)p.R) {  // uniform
    finalize_cstar(p, blockIdx.x - p.R);
    return;
  }
  __shared__ float wbuf[kMaxTiles];
  __shared__ float zbuf[kTileN];
  __shared__ float ebuf[kTileN];
  __shared__ __align__(16) T arow[kMaxRank + 16];
  __shared__ float fred[8];
  __shared__ int ired[8];
  __shared__ float s_before;
  __shared__ float2 s_ps[kMaxGamma + 1];  // (m_p, S_p) of the request's target rows
  __shared__ int s_x[kMaxGamma];          // its draft tokens
  __shared__ float s_ufin[kMaxGamma + 1];  // final-token uniform of each position

  constexpr int kTpt = kMaxTiles / kBlock;  // tiles per thread, at most
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rho = blockIdx.x, gamma = p.gamma, V = p.V, nT = p.n_tiles;
  int32_t *yrow = p.y + (int64_t)rho * (gamma + 1);

  // ---- loads that need only rho, all in flight together: the request's
  //      slice of the ragged batch (every thread validates the same values),
  //      the draft token and q(x_k) of position k = tid + 1, and the bonus
  //      row's tile partials
  const int ell_in = p.ell[rho];
  const int base_in = p.row_offset[rho];
  const int next = p.row_offset[rho + 1], rows_used = p.row_offset[p.R];
  const int32_t *xr = p.x + (int64_t)rho * gamma;
  // (unconditional loads at clamped positions: a load under a condition
  // would be waited for inside its branch)
  const int xk_raw = xr[min(tid, gamma - 1)];
  const float qk = p.q_x[(int64_t)rho * gamma + min(tid, gamma - 1)];
  const int x0 = p.x0[rho];
  float2 bt[kTpt];
#pragma unroll
  for (int i = 0; i < kTpt; ++i)
    bt[i] = p.bonus_tiles[(int64_t)rho * nT + min(tid + i * kBlock, nT - 1)];
  // an invalid slice runs as an empty one (every address stays in bounds, so
  // the loads above need not wait for the check) and is reported at the end
  const RequestSlice sl = request_slice(p, rho, ell_in, base_in, next, rows_used);
  const bool ok = sl.ok;
  const int ell = sl.ell, base = sl.base;
  const int64_t d_off = sl.d_off;

  // ---- target-row inputs of position k = tid + 1 <= ell + 1 (the row after
  //      the drafts is the bonus row): chunk statistics, and p(x_k)
  const bool own_row = tid <= ell;
  const int prow = base + (own_row ? tid : 0);
  float2 cs[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) cs[c] = p.p_chunks[(int64_t)prow * kChunks + c];
  const bool test = tid < ell;
  const int xk = xk_raw < 0 ? 0 : (xk_raw >= V ? V - 1 : xk_raw);
  const float tx = Elem<T>::at(reinterpret_cast<const T *>(p.P) + (int64_t)prow * V,
                               test ? xk : 0);

  // ---- the Philox uniforms (long integer chains) while the loads are in
  //      flight: the accept test of position k = tid + 1, and the final draw
  //      at each position it could land on (the LDS store keeps it here)
  const float u_acc = uniform01(p.seed, p.round, (uint64_t)(tid + 1), (uint64_t)rho, kStreamAccept);
  if (tid <= gamma)
    s_ufin[tid] = uniform01(p.seed, p.round, (uint64_t)(tid + 1), (uint64_t)rho, kStreamFinal);

  // ---- accept tests: u * q(x_k) < p(x_k), first rejection
  float2 ps_own = make_float2(0.0f, 0.0f);
  if (own_row) {
    ps_own = combine_chunk_stats(cs);
    s_ps[tid] = ps_own;
  }
  if (tid < gamma) s_x[tid] = xk;
  int rej = 0x7fffffff;
  if (test) {
    if (xk_raw != xk) flag_error(p.err, kErrToken);
    const int k = tid + 1;
    const double pk = exp((double)(tx * p.invT) - (double)ps_own.x) / (double)ps_own.y;
    if (!((double)u_acc * (double)qk < pk)) rej = k;
  }
  rej = block_min_int(rej, ired);  // its barriers also publish s_ps and s_x
  const int n = rej == 0x7fffffff ? ell : rej - 1;
  const int j = n + 1;             // position of the final token
  const int frow = base + n;       // its target row
  const float2 ps = s_ps[n];
  const float uf = s_ufin[n];  // position j = n + 1
  const T *Prow = reinterpret_cast<const T *>(p.P) + (int64_t)frow * V;
  int final_token = 0;

  bool residual = n < ell;
  if (residual) {
    // residual masses per tile from the verify pass; the transition row and
    // q statistics of position j load meanwhile
    const float2 *pp = p.pair_partials + (d_off + j - 1) * nT;
    float w[kTpt];
#pragma unroll
    for (int i = 0; i < kTpt; ++i) w[i] = pp[min(tid + i * kBlock, nT - 1)].y;
    const int prev = j == 1 ? min(max(x0, 0), V - 1) : s_x[j - 2];
    const T *arow_src = p.A_given != nullptr
                            ? reinterpret_cast<const T *>(p.A_given) + ((int64_t)(j - 1) * p.R + rho) * p.r
                            : reinterpret_cast<const T *>(p.W1) + (int64_t)prev * p.r;
    const int pieces = p.r * (int)sizeof(T) / 16;
    uint4 arow_piece = make_uint4(0, 0, 0, 0);
    if (tid < pieces)
      arow_piece = *reinterpret_cast<const uint4 *>(arow_src + tid * (16 / sizeof(T)));
    const int64_t qi = (int64_t)rho * gamma + j - 1;
    const float mq = p.q_stats[2 * qi], sq = p.q_stats[2 * qi + 1];
#pragma unroll
    for (int i = 0; i < kTpt; ++i)
      if (tid + i * kBlock < nT) wbuf[tid + i * kBlock] = w[i];
    if (tid < pieces) *reinterpret_cast<uint4 *>(arow + tid * (16 / sizeof(T))) = arow_piece;
    __syncthreads();
    float total, target;
    const int tstar = pick_tile(wbuf, nT, uf, fred, ired, &s_before, &total, &target);
    if (total > 0.0f) {
      const int col = tstar * kTileN + tid;
      const float tcol = tid < kTileN && col < V ? Elem<T>::at(Prow, col) : 0.0f;
      const T *Urow = reinterpret_cast<const T *>(p.U) + ((int64_t)rho * gamma + j - 1) * V;
      recompute_tile_v<T, false>(arow, reinterpret_cast<const T *>(p.W2), Urow, V, p.r, tstar,
                                 (int)((d_off + j - 1) & 31), zbuf);
      __syncthreads();
      if (tid < kTileN) {
        // (p - q)_+ = p - min(p, q), each term formed as in the verify pass
        const float lq = log2_fast(sq), lp = log2_fast(ps.y);
        float e = 0.0f;
        if (col < V) {
          const float a = log2_prob(tcol, p.invT, ps.x, lp);
          const float b = log2_prob(zbuf[tid], p.invT, mq, lq);
          e = exp2_fast(a) - exp2_fast(fminf(a, b));
        }
        ebuf[tid] = e;
      }
      __syncthreads();
      if (wave == 0) {
        const int pick = pick_in_tile(ebuf, s_before, 1.0f, target);
        if (lane == 0) ired[4] = tstar * kTileN + pick;
      }
      __syncthreads();
      final_token = ired[4];
    } else {
      residual = false;  // residual mass rounded to zero: fall back to p_j
    }
  }
  if (!residual) {
    // p_j by tiles: the bonus row has kept partials; a rejected row (fallback)
    // gets its tile masses by one pass over the row
    const bool bonus = n == ell;
    if (bonus) {
#pragma unroll
      for (int i = 0; i < kTpt; ++i) {
        const int t = tid + i * kBlock;
        if (t < nT) wbuf[t] = bt[i].y * fexp(bt[i].x - ps.x);
      }
    } else {
      for (int t = wave; t < nT; t += kBlock / kWave) {
        float acc = 0.0f;
        for (int q = lane; q < kTileN; q += kWave) {
          const int col = t * kTileN + q;
          if (col < V) acc += fexp(Elem<T>::at(Prow, col) * p.invT - ps.x);
        }
        acc = wave_sum(acc);
        if (lane == 0) wbuf[t] = acc;
      }
    }
    __syncthreads();
    float total, target;
    const int tstar = pick_tile(wbuf, nT, uf, fred, ired, &s_before, &total, &target);
    if (tid < kTileN) {
      const int col = tstar * kTileN + tid;
      ebuf[tid] = col < V ? fexp(Elem<T>::at(Prow, col) * p.invT - ps.x) : 0.0f;
    }
    __syncthreads();
    if (wave == 0) {
      const int pick = pick_in_tile(ebuf, s_before, 1.0f, target);
      if (lane == 0) ired[4] = tstar * kTileN + pick;
    }
    __syncthreads();
    final_token = ired[4];
  }

  // ---- outputs
  if (!ok) {  // uniform
    if (tid == 0) flag_error(p.err, kErrLength);
    for (int i = tid; i <= gamma; i += kBlock) yrow[i] = -1;
    if (tid == 0) p.n_acc[rho] = 0;
    return;
  }
  for (int i = tid; i <= gamma; i += kBlock) {
    int v = -1;
    if (i < n) v = xr[i];
    else if (i == n) v = final_token;
    yrow[i] = v;
  }
  if (tid == 0) p.n_acc[rho] = n;
}

bool verify_stationary_shape(int V, int r, bool bf16, int *grid, int *nt);
hipError_t launch_verify_stationary(const VerifyLaunch &L, int G, int nt, hipStream_t stream);

// Below this many possible verified rows (R gamma) the row-stationary product
// is used: it is one row group, so it reads W2 once.
constexpr int kStationaryMinRows = 256;

// DSPARK_STATIONARY_VERIFY=0 in the environment selects the row-stationary
// verify product for every shape (a switch to compare the two designs).
static bool getenv_stationary_enabled() {
  static const bool on = [] {
    const char *v = getenv("DSPARK_STATIONARY_VERIFY");
    return v == nullptr || v[0] != '0';
  }();
  return on;
}

template <typename T>
static hipError_t launch_verify_t(const VerifyLaunch &L, hipStream_t stream) {
  const int nT = n_tiles_of(L.V);
  RowStatsParams rs{};
  rs.n_rows = L.rows_capacity; rs.V = L.V; rs.n_tiles = nT; rs.invT = L.invT; rs.X = L.P;
  rs.row_offset = L.row_offset; rs.R = L.R; rs.chunks = L.p_chunks;
  rs.bonus_tiles = L.bonus_tiles; rs.err = L.err;
  rs.gamma = L.gamma; rs.x0 = L.x0; rs.x = L.x; rs.row_map = L.row_map;
  rs.r = L.r; rs.W1 = L.W1; rs.A_rows = L.A_rows; rs.A_given = L.A_given;
  // at most 1024 rows of workgroups: the rows in use are known only on the
  // device, and a grid of the host's bound (R (1 + gamma)) dispatched mostly
  // workgroups that only found they had no row (4% slower at R = 128)
  constexpr int kRowGrid = 1024;
  DSPARK_LAUNCH("row_chunk_stats", stream, row_chunk_stats_kernel<T>,
                dim3(kChunks, L.rows_capacity < kRowGrid ? L.rows_capacity : kRowGrid), kBlock, rs);

  BiasTileParams bp{};
  bp.R = L.R; bp.gamma = L.gamma; bp.V = L.V; bp.r = L.r; bp.n_tiles = nT; bp.invT = L.invT;
  bp.U = L.U; bp.W1 = L.W1; bp.W2 = L.W2; bp.x0 = L.x0; bp.x = L.x; bp.err = L.err;
  bp.ell = L.ell; bp.row_offset = L.row_offset; bp.rows_capacity = L.rows_capacity;
  bp.P = L.P; bp.p_chunks = L.p_chunks; bp.q_stats = L.q_stats; bp.pair_partials = L.pair_partials;
  bp.row_map = L.row_map;
  bp.A = L.A_rows;
  // the number of verified drafts lives on the device: each workgroup (one per
  // compute unit) takes an equal share of the (row group, tile) items it
  // finds there
  const int grid = kComputeUnits;
  int sgrid = 0, snt = 0;
  if (getenv_stationary_enabled() && L.R * L.gamma > kStationaryMinRows &&
      verify_stationary_shape(L.V, L.r, sizeof(T) == 2, &sgrid, &snt)) {
    // bf16, rank 256, more than one 256-row group possible: W2 held on chip,
    // every verified row streamed past it (verify_stationary.hip).  With at
    // most 256 verified rows the row-stationary kernel reads W2 once anyway
    // and has no prologue to hide (R = 32, gamma = 7: 51.5 against 58 us).
    const hipError_t e = launch_verify_stationary(L, sgrid, snt, stream);
    if (e != hipSuccess) return e;
  } else if (L.r == (L.bf16 ? kMaxRank : 128)) {
    // row groups of 256 rows (8 waves x 1 row block: each W2 block in LDS
    // serves twice the rows of a 4-wave group; measured faster than 4 waves
    // and than 2 or 3 row blocks per wave)
    DSPARK_LAUNCH("bias_tile_verify", stream,
                  (stream_tile_kernel<T, Epi::kVerify, sizeof(T) == 2 ? kMaxRank / 16 : 64, 8, 1>),
                  grid, 8 * kWave, bp);
  } else {
    DSPARK_LAUNCH("bias_tile_verify", stream, (stream_tile_kernel<T, Epi::kVerify, 0, 8, 1>), grid,
                  8 * kWave, bp);
  }

  FinalizeParams fp{};
  fp.R = L.R; fp.gamma = L.gamma; fp.V = L.V; fp.r = L.r; fp.n_tiles = nT; fp.A_given = L.A_given;
  fp.rows_capacity = L.rows_capacity; fp.invT = L.invT; fp.ell = L.ell; fp.row_offset = L.row_offset;
  fp.P = L.P; fp.U = L.U; fp.W1 = L.W1; fp.W2 = L.W2; fp.x0 = L.x0; fp.x = L.x;
  fp.q_stats = L.q_stats; fp.q_x = L.q_x; fp.seed = L.seed; fp.round = L.round;
  fp.p_chunks = L.p_chunks; fp.bonus_tiles = L.bonus_tiles; fp.pair_partials = L.pair_partials;
  fp.n_acc = L.n_acc; fp.y = L.y; fp.c_star = L.c_star; fp.err = L.err;
  DSPARK_LAUNCH("verify_finalize", stream, verify_finalize_kernel<T>, 2 * L.R, kBlock, fp);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyLaunch &L, hipStream_t stream) {
  return L.bf16 ? launch_verify_t<bf16_t>(L, stream) : launch_verify_t<float>(L, stream);
}

// ------------------------------------------------------------- tv_overlap
struct OverlapParams {
  int n_rows, V, n_tiles;
  float invT;
  const void *P, *Q;
  const float *p_stats, *q_stats;     // given (m, S), or NULL
  const float2 *p_chunks, *q_chunks;  // computed, when the stats are not given
  float *partial;                     // [n_rows][kChunks]
};

// sum over one quarter of a row pair of min(p, q), one workgroup per quarter:
// rounds of kBatch 16-byte pieces of P and of Q per thread, two rounds in
// flight (non-temporal loads; indices clamped, so no branch stands between
// the loads: past the chunk they read its last piece again and the results
// are not used), the row's statistics loaded behind the first two rounds.
// min(p, q) = 2^min(log2 p, log2 q): one exponential per element.
template <typename T>
__global__ __launch_bounds__(kBlock) void overlap_chunk_kernel(OverlapParams p) {
  __shared__ float red[8];
  constexpr int kPer = Elem<T>::kPerVec;
  constexpr int kBatch = 2;
  constexpr int kRound = kBatch * kBlock;
  const int c = blockIdx.x, tid = threadIdx.x, V = p.V, nT = p.n_tiles;
  const int tpc = (nT + kChunks - 1) / kChunks;
  // an empty chunk starts at V (its clamped loads read the row's last piece)
  const int vb = min(min(c * tpc, nT) * kTileN, V), ve = min(min(c * tpc + tpc, nT) * kTileN, V);
  const int npc = (ve - vb + kPer - 1) / kPer;  // pieces in the chunk (V % kPer == 0)
  const float invT = p.invT;
  // rows blockIdx.y, blockIdx.y + gridDim.y, ... (the grid's second
  // dimension is capped)
  for (int row = blockIdx.y; row < p.n_rows; row += gridDim.y) {
    const T *Pr = reinterpret_cast<const T *>(p.P) + (int64_t)row * V + vb;
    const T *Qr = reinterpret_cast<const T *>(p.Q) + (int64_t)row * V + vb;
    auto issue = [&](u32x4 (&a)[kBatch], u32x4 (&b)[kBatch], int p0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int64_t off = (int64_t)min(p0 + j * kBlock + tid, npc - 1) * kPer;
        a[j] = ld_stream4(Pr + off);
        b[j] = ld_stream4(Qr + off);
      }
    };
    u32x4 ca[kBatch], cb[kBatch], na[kBatch], nb[kBatch];
    issue(ca, cb, 0);
    issue(na, nb, kRound);
    float mp, lp, mq, lq;  // (m, log2 S) of p and of q
    if (p.p_stats != nullptr) {
      mp = p.p_stats[2 * (int64_t)row]; lp = log2_fast(p.p_stats[2 * (int64_t)row + 1]);
      mq = p.q_stats[2 * (int64_t)row]; lq = log2_fast(p.q_stats[2 * (int64_t)row + 1]);
    } else {
      const float2 a = combine_chunk_stats(p.p_chunks + (int64_t)row * kChunks);
      const float2 b = combine_chunk_stats(p.q_chunks + (int64_t)row * kChunks);
      mp = a.x; lp = log2_fast(a.y); mq = b.x; lq = log2_fast(b.y);
    }
    float acc = 0.0f;
    auto reduce = [&](const u32x4 (&a)[kBatch], const u32x4 (&b)[kBatch], int p0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float x[kPer], y[kPer];
        unpack16(a[j], (T *)nullptr, x);
        unpack16(b[j], (T *)nullptr, y);
        float sj = 0.0f;
#pragma unroll
        for (int q = 0; q < kPer; ++q)
          sj += exp2_fast(fminf(log2_prob(x[q], invT, mp, lp), log2_prob(y[q], invT, mq, lq)));
        acc += p0 + j * kBlock + tid < npc ? sj : 0.0f;
      }
    };
    for (int p0 = 0; p0 < npc; p0 += 2 * kRound) {
      reduce(ca, cb, p0);
      issue(ca, cb, p0 + 2 * kRound);
      if (p0 + kRound < npc) reduce(na, nb, p0 + kRound);
      issue(na, nb, p0 + 3 * kRound);
    }
    const float s = block_sum(acc, red);
    if (tid == 0) p.partial[(int64_t)row * kChunks + c] = s;
  }
}

__global__ void overlap_combine_kernel(int n_rows, const float *partial, float *c_star) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) s += partial[(int64_t)row * kChunks + c];
  c_star[row] = s;
}

template <typename T>
static hipError_t launch_overlap_t(const OverlapLaunch &L, hipStream_t stream) {
  const int nT = n_tiles_of(L.V);
  // the grid's second dimension is at most 65535; past it the kernels loop
  const int gy = L.n_rows < 65535 ? L.n_rows : 65535;
  if (L.p_stats == nullptr) {
    RowStatsParams rs{};
    rs.n_rows = L.n_rows; rs.V = L.V; rs.n_tiles = nT; rs.invT = L.invT; rs.err = L.err;
    rs.X = L.P; rs.chunks = L.p_chunks;
    DSPARK_LAUNCH("row_chunk_stats", stream, row_chunk_stats_kernel<T>, dim3(kChunks, gy), kBlock, rs);
    rs.X = L.Q; rs.chunks = L.q_chunks;
    DSPARK_LAUNCH("row_chunk_stats", stream, row_chunk_stats_kernel<T>, dim3(kChunks, gy), kBlock, rs);
  }
  OverlapParams op{};
  op.n_rows = L.n_rows; op.V = L.V; op.n_tiles = nT; op.invT = L.invT; op.P = L.P; op.Q = L.Q;
  op.p_stats = L.p_stats; op.q_stats = L.q_stats; op.p_chunks = L.p_chunks;
  op.q_chunks = L.q_chunks; op.partial = L.partial;
  DSPARK_LAUNCH("overlap_chunk", stream, overlap_chunk_kernel<T>, dim3(kChunks, gy), kBlock, op);
  DSPARK_LAUNCH("overlap_combine", stream, overlap_combine_kernel, (L.n_rows + 255) / 256, 256,
                L.n_rows, L.partial, L.c_star);
  return hipGetLastError();
}

hipError_t launch_overlap(const OverlapLaunch &L, hipStream_t stream) {
  return L.bf16 ? launch_overlap_t<bf16_t>(L, stream) : launch_overlap_t<float>(L, stream);
}

__global__ void clear_error_kernel(int32_t *err) { *err = 0; }

hipError_t launch_clear_error(int32_t *err, hipStream_t stream) {
  clear_error_kernel<<<1, 1, 0, stream>>>(err);
  return hipGetLastError();
}

}  // namespace dspark
