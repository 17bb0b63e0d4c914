// Markov-head drafting (Blog, "Markov sequential head"; Bangkok 4.1; KB
// section 2): gamma serial steps.  For bf16, rank 256 and up to 512 requests
// all of them run in one cooperative launch that keeps W2 on chip
// (draft_persistent.hip); otherwise (and when that launch is refused) each
// step is one fused bias-tile launch (partials of z_k per vocabulary tile) +
// one sampling launch (one workgroup per request, the two-level inverse CDF
// of sampler.h), and the recurrent head adds its state update per step.
//
// The transition rows W1[x_{k-1}] of step k > 1 sit in a contiguous [R][r]
// buffer (A_k) written by the sampler of step k-1, so the tile kernel loads
// them together with its W2 columns and U rows, with no dependent token lookup
// in between; step 1 reads W1[x0] in place (the anchors are known before the
// launch, and the first launch saves a gather kernel).
#include <stdlib.h>

#include "bias_tile.h"
#include "kernels.h"
#include "sampler.h"
#include "trace.h"

namespace dspark {

// DSPARK_PERSISTENT_DRAFT=0 in the environment selects the per-step kernels
// for every shape (a switch to compare the two designs on one workload).
static bool getenv_persistent_enabled() {
  static const bool on = [] {
    const char *v = getenv("DSPARK_PERSISTENT_DRAFT");
    return v == nullptr || v[0] != '0';
  }();
  return on;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void draft_sample_kernel(SampleParams p) {
  __shared__ SampleLds sl;
  __shared__ __align__(16) T arow[kMaxRank + 16];
  sample_row<T>(p, p.k, p.A_next, blockIdx.x, arow, true, sl);
}

// sh[rho][k] = sum_j w[j] h[rho][k][j]: one wave per (rho, k).  Lane l takes
// the 16-byte pieces l, l + 64, ... of the row in that order, kIt of them in
// flight at a time (non-temporal loads of h, read once; indices clamped, so
// no branch stands between the loads), with their kPer weights each.
template <typename T>
__global__ __launch_bounds__(kBlock) void head_hidden_dot_kernel(int n_slots, int d,
                                                                 const T *h, const float *w,
                                                                 float *sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t slot = (int64_t)blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (slot >= n_slots) return;
  constexpr int kPer = Elem<T>::kPerVec;  // elements per 16-byte piece
  constexpr int kIt = 8;
  const T *row = h + slot * d;
  const int np = d / kPer;  // d % 8 == 0
  float acc = 0.0f;
  for (int p0 = 0; p0 < np; p0 += kIt * kWave) {
    u32x4 v[kIt];
    float4 wv[kIt][kPer / 4];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int pc = min(p0 + i * kWave + lane, np - 1);
      v[i] = ld_stream4(row + (int64_t)pc * kPer);
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) wv[i][q] = reinterpret_cast<const float4 *>(w + pc * kPer)[q];
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      if (p0 + i * kWave + lane < np) {
        float hv[kPer];
        unpack16(v[i], (T *)nullptr, hv);
#pragma unroll
        for (int q = 0; q < kPer / 4; ++q) {
          acc = fmaf(wv[i][q].x, hv[4 * q], acc);
          acc = fmaf(wv[i][q].y, hv[4 * q + 1], acc);
          acc = fmaf(wv[i][q].z, hv[4 * q + 2], acc);
          acc = fmaf(wv[i][q].w, hv[4 * q + 3], acc);
        }
      }
    }
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

bool persistent_draft_shape(int R, int V, int r, bool bf16, int *grid, int *nt);
hipError_t launch_draft_persistent(const DraftLaunch &L, int G, int nt, const SampleParams &sp,
                                   hipStream_t stream);

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
  // bf16, rank 256, up to 512 requests: every step in one persistent launch
  // that keeps W2 on chip (draft_persistent.hip)
  int pgrid = 0, pnt = 0;
  if (L.rnn == nullptr && getenv_persistent_enabled() &&
      persistent_draft_shape(L.R, L.V, L.r, sizeof(T) == 2, &pgrid, &pnt)) {
    hipError_t e = launch_draft_persistent(L, pgrid, pnt, sp, stream);
    if (e == hipSuccess) return hipGetLastError();
    (void)hipGetLastError();  // not co-resident on this device: per-step kernels below
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
