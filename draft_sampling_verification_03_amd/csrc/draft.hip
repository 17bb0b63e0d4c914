// Markov-head drafting (Blog, "Markov sequential head"; Bangkok 4.1; KB
// section 2): gamma serial steps, each = one fused bias-tile launch (partials
// of z_k per vocabulary tile) + one sampling launch (one workgroup per request).
//
// Sampling is an inverse CDF in two levels.  The workgroup of request rho
// rescales its tile partials to the row maximum, scans them to find the tile
// whose cumulative mass first exceeds u * S, recomputes z for that tile alone
// (bit-identical to the fused kernel), and scans inside the tile.  Only the
// 128-column tile is re-read, never the row.
//
// The transition rows W1[x_{k-1}] of step k > 1 sit in a contiguous [R][r]
// buffer (A_k) written by the sampler of step k-1, so the tile kernel loads
// them together with its W2 columns and U rows, with no dependent token lookup
// in between; step 1 reads W1[x0] in place (the anchors are known before the
// launch, and the first launch saves a gather kernel).
#include "bias_tile.h"
#include "kernels.h"
#include "trace.h"

namespace dspark {

struct SampleParams {
  int R, gamma, V, r, n_tiles, k;
  float invT;
  const void *U, *W1, *W2;
  const void *A_cur;         // [R][r]: W1[x_{k-1}] of every request
  const int32_t *a_tokens;   // or, if set, x_{k-1} (A_cur row rho = W1[a_tokens[rho]])
  void *A_next;              // [R][r]: receives W1[x_k] (NULL at the last step)
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

template <typename T>
__global__ __launch_bounds__(kBlock) void draft_sample_kernel(SampleParams p) {
  constexpr int kCpt = kMaxTiles / kBlock;  // tiles per thread, at most
  __shared__ float zbuf[kTileN];
  __shared__ __align__(16) T arow[kMaxRank + 16];
  __shared__ float red_max[4], red_sum[4];
  __shared__ int red_found[4], red_last[4];
  __shared__ float s_before, s_mt, s_u;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int rho = blockIdx.x, k = p.k, V = p.V, r = p.r, nT = p.n_tiles;
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
    if (tid < pieces) a = *reinterpret_cast<const uint4 *>(Acur + tid * kPer);
    const float2 *ts = p.tile_stats + (int64_t)rho * nT;
#pragma unroll
    for (int j = 0; j < kCpt; ++j) pt[j] = t0 + j < t1 ? ts[t0 + j] : make_float2(-INFINITY, 0.0f);
    // the draw's uniform (a scalar Philox chain) is formed while the loads
    // are in flight: the LDS store keeps it ahead of the first barrier
    if (tid == 0) s_u = uniform01(p.seed, p.round, (uint64_t)k, (uint64_t)rho, kStreamDraft);
    if (tid < pieces) *reinterpret_cast<uint4 *>(arow + tid * kPer) = a;
  }
  // 2. row maximum, then tile masses w_t = s_t exp(m_t - m) and their
  //    exclusive scan in tile order (one barrier each)
  float lm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kCpt; ++j) lm = fmaxf(lm, pt[j].x);
  lm = wave_max(lm);
  if (lane == 0) red_max[wave] = lm;
  __syncthreads();
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
  recompute_tile_v<T, true>(arow, reinterpret_cast<const T *>(p.W2), Urow, V, r, tstar, rho & 31,
                            zbuf);
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
    if (lane == 0) {
      p.x[slot] = finite ? xk : -1;
      p.q_stats[2 * slot] = m;
      p.q_stats[2 * slot + 1] = S;
      p.q_x[slot] = fexp(zp - m) / S;
      if (p.logq_x != nullptr) p.logq_x[slot] = (zp - m) - logf(S);
    }
    // 7. the next step's transition row A_{k+1}[rho] = W1[x_k], by this wave
    //    (no barrier: the token is in its registers)
    if (p.A_next != nullptr && lane < pieces) {
      const int xc = min(max(xk, 0), V - 1);
      *reinterpret_cast<uint4 *>(reinterpret_cast<T *>(p.A_next) + (int64_t)rho * r + lane * kPer) =
          *reinterpret_cast<const uint4 *>(reinterpret_cast<const T *>(p.W1) + (int64_t)xc * r +
                                           lane * kPer);
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
}

// sh[rho][k] = sum_j w[j] h[rho][k][j]: one wave per (rho, k), 16-byte loads.
template <typename T>
__global__ __launch_bounds__(kBlock) void head_hidden_dot_kernel(int n_slots, int d,
                                                                 const T *h, const float *w,
                                                                 float *sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t slot = (int64_t)blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (slot >= n_slots) return;
  constexpr int kPer = Elem<T>::kPerVec;
  const T *row = h + slot * d;
  float acc = 0.0f;
  for (int j = lane * kPer; j < d; j += kWave * kPer) {
    float hv[kPer];
    Elem<T>::vec(row, j, hv);
#pragma unroll
    for (int q = 0; q < kPer; ++q) acc = fmaf(w[j + q], hv[q], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) sh[slot] = acc;
}

// Recurrent head (Blog "RNN sequential head"; KB section 3), the gated update
// read as a GRU:
//   g = G_E[x_{k-1}] + G_h[rho][k-1];  a = W_hh s_{k-1} + b_hh
//   s_k = (1 - sigmoid(g_z + a_z)) tanh(g_n + sigmoid(g_r + a_r) a_n)
//         + sigmoid(g_z + a_z) s_{k-1}
// a = W_hh s is a small product [R x r] x [r x 3r] over the column-major
// weights (393 KB at r = 256 bf16, L2-resident).  A workgroup takes 4
// requests x 64 state units (the three gate columns of each unit), so every
// weight it loads serves 4 requests and the grid has R/4 x r/64 workgroups.
// Thread (og, sp) owns 16 bytes of output columns og and a contiguous range
// sp of the inputs: one coalesced 16-byte load per input row, up to 16 input
// ranges so the dependent load chain stays short, and each thread issues its
// rows' loads 8 at a time before using any (the kernel is bound by load
// latency); the ranges' partial sums meet in LDS in a fixed order.  s_k is
// kept in fp32; the product's transition row A_k = s_k in the weights' type.
struct GruParams {
  int R, gamma, V, r, k;
  const void *G_E;     // [V][3r]
  const float *G_h;    // [R][gamma][3r]
  const void *W_hh;    // [r][3r]
  const float *b_hh;   // [3r]
  const int32_t *x0, *x;
  const float *s0;     // [R][r] or NULL (zeros)
  float *s;            // [R][gamma][r]
  void *A;             // [gamma][R][r]
  int32_t *err;
};

constexpr int kGruReq = 4, kGruUnits = 64, kGruSplits = 16, kGruBlock = 512, kGruBatch = 8;

template <typename T>
__global__ __launch_bounds__(kGruBlock) void gru_step_kernel(GruParams p) {
  constexpr int kPer = 16 / (int)sizeof(T);
  __shared__ float sprev[kGruReq][kMaxRank];
  __shared__ float apart[kGruSplits][kGruReq][3 * kGruUnits];
  const int tid = threadIdx.x, r = p.r, g3 = 3 * r, k = p.k;
  const int rho0 = blockIdx.x * kGruReq;
  const int nu = min(r, kGruUnits), u0 = blockIdx.y * nu;
  // the combining thread's input pre-activations g load first, so their
  // latency (token, then embedding row) overlaps the product below
  const int cq = tid / nu, cj = u0 + tid % nu, crho = rho0 + cq;
  const bool combiner = tid < kGruReq * nu && crho < p.R && cj < r;
  float gr = 0.0f, gz = 0.0f, gn = 0.0f;
  if (combiner) {
    int prev = k == 1 ? p.x0[crho] : p.x[(int64_t)crho * p.gamma + k - 2];
    if (prev < 0 || prev >= p.V) {
      if (cj == u0) flag_error(p.err, kErrToken);
      prev = min(max(prev, 0), p.V - 1);
    }
    const T *ge = reinterpret_cast<const T *>(p.G_E) + (int64_t)prev * g3;
    const float *gh = p.G_h + ((int64_t)crho * p.gamma + k - 1) * g3;
    gr = Elem<T>::at(ge, cj) + gh[cj];
    gz = Elem<T>::at(ge, r + cj) + gh[r + cj];
    gn = Elem<T>::at(ge, 2 * r + cj) + gh[2 * r + cj];
  }
  for (int idx = tid; idx < kGruReq * r; idx += kGruBlock) {
    const int q = idx / r, i = idx % r, rho = rho0 + q;
    float v = 0.0f;
    if (rho < p.R) {
      if (k > 1) v = p.s[((int64_t)rho * p.gamma + k - 2) * r + i];
      else if (p.s0 != nullptr) v = p.s0[(int64_t)rho * r + i];
    }
    sprev[q][i] = v;
  }
  __syncthreads();
  const int ppg = nu / kPer;        // 16-byte pieces per gate
  const int groups = 3 * ppg;
  const int nsplit = min(kGruSplits, kGruBlock / groups);
  const int per = (r + nsplit - 1) / nsplit;
  if (tid < groups * nsplit) {
    const int og = tid % groups, sp = tid / groups;
    const int gate = og / ppg, pc = og % ppg;
    const int unit = u0 + pc * kPer;  // a piece is wholly inside [0, r) or wholly outside
    float acc[kGruReq][kPer];
#pragma unroll
    for (int q = 0; q < kGruReq; ++q)
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[q][e] = 0.0f;
    const int i0 = sp * per, i1 = min(r, i0 + per);
    if (unit < r && i0 < i1) {
      const T *W = reinterpret_cast<const T *>(p.W_hh) + gate * r + unit;
      // batches of kGruBatch rows: all their loads issue before the first is
      // used (rows past the range re-read the last one and count with weight 0)
      for (int ib = i0; ib < i1; ib += kGruBatch) {
        uint4 raw[kGruBatch];
#pragma unroll
        for (int u = 0; u < kGruBatch; ++u)
          raw[u] = *reinterpret_cast<const uint4 *>(W + (int64_t)min(ib + u, i1 - 1) * g3);
#pragma unroll
        for (int u = 0; u < kGruBatch; ++u) {
          float w[kPer];
          const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
          if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __uint_as_float(wd[e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              w[2 * e] = __uint_as_float(wd[e] << 16);
              w[2 * e + 1] = __uint_as_float(wd[e] & 0xffff0000u);
            }
          }
          const bool in = ib + u < i1;
#pragma unroll
          for (int q = 0; q < kGruReq; ++q) {
            const float si = in ? sprev[q][min(ib + u, i1 - 1)] : 0.0f;
#pragma unroll
            for (int e = 0; e < kPer; ++e) acc[q][e] = fmaf(w[e], si, acc[q][e]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kGruReq; ++q)
#pragma unroll
      for (int e = 0; e < kPer; ++e) apart[sp][q][gate * nu + pc * kPer + e] = acc[q][e];
  }
  __syncthreads();
  if (!combiner) return;
  const int q = cq, jj = tid % nu, j = cj, rho = crho;
  float ar = p.b_hh[j], az = p.b_hh[r + j], an = p.b_hh[2 * r + j];
  for (int sp = 0; sp < nsplit; ++sp) {
    ar += apart[sp][q][jj];
    az += apart[sp][q][nu + jj];
    an += apart[sp][q][2 * nu + jj];
  }
  const float rg = 1.0f / (1.0f + expf(-(gr + ar)));
  const float zg = 1.0f / (1.0f + expf(-(gz + az)));
  const float n = tanhf(gn + rg * an);
  const float sk = (1.0f - zg) * n + zg * sprev[q][j];
  p.s[((int64_t)rho * p.gamma + k - 1) * r + j] = sk;
  store_elem(reinterpret_cast<T *>(p.A), ((int64_t)(k - 1) * p.R + rho) * r + j, sk);
}

template <typename T, int KS>
static hipError_t launch_draft_t(const DraftLaunch &L, hipStream_t stream) {
  const int n_tiles = (L.V + kTileN - 1) / kTileN;
  BiasTileParams bp{};
  bp.R = L.R; bp.gamma = L.gamma; bp.V = L.V; bp.r = L.r; bp.n_tiles = n_tiles;
  bp.invT = L.invT; bp.U = L.U; bp.W1 = L.W1; bp.W2 = L.W2; bp.x0 = L.x0; bp.x = L.x;
  bp.err = L.err; bp.tile_stats = L.tile_stats;
  SampleParams sp{};
  sp.R = L.R; sp.gamma = L.gamma; sp.V = L.V; sp.r = L.r; sp.n_tiles = n_tiles;
  sp.invT = L.invT; sp.U = L.U; sp.W1 = L.W1; sp.W2 = L.W2; sp.x = L.x;
  sp.q_stats = L.q_stats; sp.q_x = L.q_x; sp.tile_stats = L.tile_stats;
  sp.seed = L.seed; sp.round = L.round; sp.err = L.err;
  sp.x_force = L.x_force; sp.logq_x = L.logq_x;
  if (L.h != nullptr) {
    const int n_slots = L.R * L.gamma;
    DSPARK_LAUNCH("head_hidden_dot", stream, head_hidden_dot_kernel<T>, (n_slots + 3) / 4, kBlock,
                  n_slots, L.d, reinterpret_cast<const T *>(L.h), L.w_conf, L.sh);
    sp.sh = L.sh; sp.w_e = L.w_conf + L.d; sp.b_conf = L.b_conf; sp.c = L.c;
    sp.conf_temp = L.conf_temp;
  }
  // the first step reads its transition rows W1[x0] in place; the sampler of
  // step k writes W1[x_k] contiguously for step k + 1
  void *A[2] = {L.A0, L.A1};
  // row groups of 32 NW requests x vocabulary tiles, in equal contiguous ranges
  // over one workgroup per compute unit: 4 waves up to 128 requests, else 8
  const bool wide = L.R > 4 * kRowsPerWave;
  const int n_items = (L.R + (wide ? 8 : 4) * kRowsPerWave - 1) / ((wide ? 8 : 4) * kRowsPerWave) * n_tiles;
  const int grid = stream_tile_grid(n_items, kComputeUnits);
  GruParams gp{};
  const int gru_units = L.r < kGruUnits ? L.r : kGruUnits;
  const dim3 gru_grid((L.R + kGruReq - 1) / kGruReq, (L.r + gru_units - 1) / gru_units);
  if (L.rnn != nullptr) {
    const RnnHead &h = *L.rnn;
    gp.R = L.R; gp.gamma = L.gamma; gp.V = L.V; gp.r = L.r; gp.G_E = h.G_E; gp.G_h = h.G_h;
    gp.W_hh = h.W_hh; gp.b_hh = h.b_hh; gp.x0 = L.x0; gp.x = L.x; gp.s0 = h.s0; gp.s = h.s;
    gp.A = h.A; gp.err = L.err;
  }
  for (int k = 1; k <= L.gamma; ++k) {
    bp.k = k;
    bp.A = A[(k - 1) & 1];
    bp.a_tokens = k == 1 ? L.x0 : nullptr;
    sp.k = k;
    sp.A_cur = A[(k - 1) & 1];
    sp.a_tokens = k == 1 ? L.x0 : nullptr;
    sp.A_next = k < L.gamma ? A[k & 1] : nullptr;
    if (L.rnn != nullptr) {
      // the state update of step k gives the transition rows of step k
      gp.k = k;
      DSPARK_LAUNCH("gru_step", stream, gru_step_kernel<T>, gru_grid, kGruBlock, gp);
      void *Ak = reinterpret_cast<T *>(L.rnn->A) + (int64_t)(k - 1) * L.R * L.r;
      bp.A = Ak; bp.a_tokens = nullptr;
      sp.A_cur = Ak; sp.a_tokens = nullptr; sp.A_next = nullptr;
    }
    if (wide) {
      DSPARK_LAUNCH("bias_tile_draft", stream, (stream_tile_kernel<T, Epi::kDraft, KS, 8, 1>), grid,
                    8 * kWave, bp);
    } else {
      DSPARK_LAUNCH("bias_tile_draft", stream, (stream_tile_kernel<T, Epi::kDraft, KS, 4, 1>), grid,
                    4 * kWave, bp);
    }
    DSPARK_LAUNCH("draft_sample", stream, draft_sample_kernel<T>, L.R, kBlock, sp);
  }
  return hipGetLastError();
}

hipError_t launch_draft(const DraftLaunch &L, hipStream_t stream) {
  // the full rank gets a product with its K steps fixed at compile time
  if (L.bf16) {
    if (L.r == kMaxRank) return launch_draft_t<bf16_t, kMaxRank / 16>(L, stream);
    return launch_draft_t<bf16_t, 0>(L, stream);
  }
  if (L.r == 128) return launch_draft_t<float, 64>(L, stream);
  return launch_draft_t<float, 0>(L, stream);
}

}  // namespace dspark
