// Fused Markov-bias tile kernel: gather W1 rows -> matrix-core product with W2
// -> add U_k and scale by 1/T -> per-(row, vocabulary tile) reduction.
//
// The pages' Markov head (Blog, "Markov sequential head"; KB section 2) adds
// the bias row W1[x_{k-1}, :] W2 to the backbone logits U_k.  For a batch of
// rows this is an [M, r] x [r, V] product whose only consumer is a
// vocabulary-wide reduction, so z is never written to HBM: each workgroup owns
// TM rows x 128 columns, keeps the tile on chip and emits one partial per row.
//
//   Draft epilogue  (m_t, s_t) = (max_v z, sum_v exp(z - m_t)) of the tile
//   Verify epilogue (sum_v min(p, q), sum_v (p - q)_+) of the tile, with
//                   q = exp(z - m_q)/S_q from the draft's statistics and
//                   p = exp(t/T - m_p)/S_p from the target row statistics
//
// Work split: 4 waves; TM = 128 -> 2 x 2 waves of 64 x 64; TM = 64 -> 1 x 4
// waves of 64 x 32; TM = 32 -> 1 x 4 waves of 32 x 32.  A (gathered W1 rows)
// is staged in LDS; B (W2 columns, r contiguous coefficients each) is read by
// every wave straight into matrix-core operand registers.  The accumulator
// tile is transposed through the same LDS region for a row-wise epilogue in
// which each thread owns TM*128/256 consecutive columns of one row, so U and
// P are read with 16-byte loads along the row.
#pragma once
#include "common.h"

namespace dspark {

constexpr int kLdsBytesPerRow = 528;  // max(r_max + 8 bf16, r_max + 4 f32, 132 f32)
constexpr int kChunks = 4;            // target-row statistics are kept per quarter row

template <int TM> struct TileShape;
template <> struct TileShape<128> { static constexpr int WM = 2, WN = 2, WMB = 2, WNB = 2; };
template <> struct TileShape<64> { static constexpr int WM = 1, WN = 4, WMB = 2, WNB = 1; };
template <> struct TileShape<32> { static constexpr int WM = 1, WN = 4, WMB = 1, WNB = 1; };

// Combined statistics of one target row from its kChunks partials, in chunk
// order.  Every consumer calls this, so all see the same (m_p, S_p).
__device__ __forceinline__ float2 combine_chunk_stats(const float2 *cs) {
  float m = cs[0].x;
#pragma unroll
  for (int c = 1; c < kChunks; ++c) m = fmaxf(m, cs[c].x);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) s += cs[c].y * (cs[c].x == -INFINITY ? 0.0f : fexp(cs[c].x - m));
  return make_float2(m, s);
}

struct BiasTileParams {
  int R, gamma, V, r, n_tiles;
  float invT;
  const void *U;        // [R][gamma][V]
  const void *W1;       // [V][r]
  const void *W2;       // column-major r x V
  const int32_t *x0;    // [R]
  const int32_t *x;     // [R][gamma]
  int32_t *err;
  // draft: rows are requests at position k
  int k;
  float2 *tile_stats;   // [R][n_tiles]
  // verify: rows are the compacted verified drafts
  const int32_t *ell, *row_offset;
  int rows_capacity;
  const void *P;            // [rows_capacity][V]
  const float2 *p_chunks;   // [rows_capacity][kChunks]
  const float *q_stats;     // [R][gamma][2]
  float2 *pair_partials;    // [R*gamma][n_tiles] (sum min, sum residual)
};

enum class Epi { kDraft, kVerify };

template <typename T, int TM, Epi E>
__global__ __launch_bounds__(kBlock, 2) void bias_tile_kernel(BiasTileParams p) {
  using Sh = TileShape<TM>;
  constexpr int kG = kBlock / TM;             // threads per epilogue row
  constexpr int kSeg = TM * kTileN / kBlock;  // columns per thread
  constexpr int kPitchC = kTileN + 4;         // fp32 pitch of the transposed tile
  __shared__ __align__(16) unsigned char smem[TM * kLdsBytesPerRow];
  __shared__ int row_prev[TM];       // token whose W1 row feeds the row (-1: padding row)
  __shared__ int row_req[TM];        // request of the row
  __shared__ int row_pos[TM];        // draft position k of the row
  __shared__ int row_out[TM];        // output row index

  const int tid = threadIdx.x;
  const int mt = blockIdx.x, nt = blockIdx.y;
  const int V = p.V, r = p.r;

  // ---- rows of this tile
  int n_rows_total;
  if constexpr (E == Epi::kDraft) {
    n_rows_total = p.R;
  } else {
    n_rows_total = p.row_offset[p.R] - p.R;  // sum of ell
    if (n_rows_total > p.R * p.gamma) n_rows_total = p.R * p.gamma;
  }
  if (mt * TM >= n_rows_total) return;  // uniform across the workgroup
  if (tid < TM) {
    const int i = mt * TM + tid;
    int prev = -1, rho = 0, k = 0;
    if (i < n_rows_total) {
      if constexpr (E == Epi::kDraft) {
        rho = i;
        k = p.k;
      } else {
        // request of compact row i: the last rho with row_offset[rho] - rho <= i
        int lo = 0, hi = p.R;  // invariant: d_off(lo) <= i < d_off(hi) (d_off(R) = sum ell)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (p.row_offset[mid] - mid <= i) lo = mid; else hi = mid;
        }
        rho = lo;
        k = i - (p.row_offset[rho] - rho) + 1;
        const int prow = p.row_offset[rho] + k - 1;
        if (k < 1 || k > p.gamma || k > p.ell[rho] || prow < 0 || prow >= p.rows_capacity) {
          flag_error(p.err, kErrLength);
          k = 0;  // skipped below
        }
      }
      if (k >= 1) {
        prev = k == 1 ? p.x0[rho] : p.x[(int64_t)rho * p.gamma + k - 2];
        if (prev < 0 || prev >= V) {
          flag_error(p.err, kErrToken);
          prev = prev < 0 ? 0 : V - 1;
        }
      }
    }
    row_prev[tid] = prev;
    row_req[tid] = rho;
    row_pos[tid] = k;
    row_out[tid] = i;
  }
  __syncthreads();

  // ---- gather A = W1[prev] rows into LDS (zero rows for padding)
  T *ldsA = reinterpret_cast<T *>(smem);
  const int a_pitch = lds_pitch<T>(r);
  {
    const int pieces = r * (int)sizeof(T) / 16;
    const T *W1 = reinterpret_cast<const T *>(p.W1);
    for (int idx = tid; idx < TM * pieces; idx += kBlock) {
      const int row = idx / pieces, pc = idx - row * pieces;
      uint4 v = make_uint4(0, 0, 0, 0);
      const int prev = row_prev[row];
      if (prev >= 0) v = *reinterpret_cast<const uint4 *>(W1 + (int64_t)prev * r + pc * (16 / sizeof(T)));
      *reinterpret_cast<uint4 *>(ldsA + row * a_pitch + pc * (16 / sizeof(T))) = v;
    }
  }
  __syncthreads();

  // ---- matrix cores: acc = A * W2[:, tile]
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const int wm = wave / Sh::WN, wn = wave % Sh::WN;
  floatx16 acc[Sh::WMB][Sh::WNB];
  bias_mainloop<Sh::WMB, Sh::WNB>(ldsA, a_pitch, wm * Sh::WMB * 32,
                                  reinterpret_cast<const T *>(p.W2), V, r,
                                  nt * kTileN + wn * Sh::WNB * 32, acc);
  __syncthreads();  // A no longer needed: reuse LDS for the transposed tile

  float *ldsC = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int mb = 0; mb < Sh::WMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < Sh::WNB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * Sh::WMB * 32 + mb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = wn * Sh::WNB * 32 + nb * 32 + (lane & 31);
        ldsC[row * kPitchC + col] = acc[mb][nb][e];
      }
  __syncthreads();

  // ---- row-wise epilogue
  const int erow = tid / kG;              // row of the tile
  const int c0 = (tid % kG) * kSeg;       // first column of the thread's segment
  const int k = row_pos[erow];
  const bool live = row_prev[erow] >= 0 && k >= 1;
  const int rho = row_req[erow];
  const int vbase = nt * kTileN + c0;
  const T *Urow = reinterpret_cast<const T *>(p.U) + ((int64_t)rho * p.gamma + (k >= 1 ? k - 1 : 0)) * V;
  constexpr int kPer = Elem<T>::kPerVec;

  if constexpr (E == Epi::kDraft) {
    float z[kSeg];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kSeg; j += kPer) {
      float u[kPer];
      const int v0 = vbase + j;
      if (live && v0 + kPer <= V) {
        Elem<T>::vec(Urow, v0, u);
      } else {
#pragma unroll
        for (int q = 0; q < kPer; ++q) u[q] = (live && v0 + q < V) ? Elem<T>::at(Urow, v0 + q) : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const float zz = (ldsC[erow * kPitchC + c0 + j + q] + u[q]) * p.invT;
        z[j + q] = (v0 + q < V) ? zz : -INFINITY;
        mx = fmaxf(mx, z[j + q]);
      }
    }
    mx = group_max<kG>(mx);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kSeg; ++j) s += fexp(z[j] - mx);
    s = group_sum<kG>(s);
    if (live && (tid % kG) == 0)
      p.tile_stats[(int64_t)row_out[erow] * p.n_tiles + nt] = make_float2(mx, s);
  } else {
    // draft statistics of (rho, k) and target statistics of its verify row
    float mq = 0.0f, rq = 0.0f, mp = 0.0f, rp = 0.0f;
    const T *Prow = reinterpret_cast<const T *>(p.P);
    if (live) {
      const int64_t qi = (int64_t)rho * p.gamma + k - 1;
      mq = p.q_stats[2 * qi];
      rq = 1.0f / p.q_stats[2 * qi + 1];
      const int prow = p.row_offset[rho] + k - 1;
      const float2 ps = combine_chunk_stats(p.p_chunks + (int64_t)prow * kChunks);
      mp = ps.x;
      rp = 1.0f / ps.y;
      Prow += (int64_t)prow * V;
    }
    float smin = 0.0f, sres = 0.0f;
#pragma unroll
    for (int j = 0; j < kSeg; j += kPer) {
      float u[kPer], t[kPer];
      const int v0 = vbase + j;
      if (live && v0 + kPer <= V) {
        Elem<T>::vec(Urow, v0, u);
        Elem<T>::vec(Prow, v0, t);
      } else {
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const bool ok = live && v0 + q < V;
          u[q] = ok ? Elem<T>::at(Urow, v0 + q) : 0.0f;
          t[q] = ok ? Elem<T>::at(Prow, v0 + q) : 0.0f;
        }
      }
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        if (v0 + q < V) {
          const float zz = (ldsC[erow * kPitchC + c0 + j + q] + u[q]) * p.invT;
          const float qv = fexp(zz - mq) * rq;
          const float pv = fexp(t[q] * p.invT - mp) * rp;
          smin += fminf(pv, qv);
          sres += fmaxf(pv - qv, 0.0f);
        }
      }
    }
    smin = group_sum<kG>(smin);
    sres = group_sum<kG>(sres);
    if (live && (tid % kG) == 0)
      p.pair_partials[(int64_t)row_out[erow] * p.n_tiles + nt] = make_float2(smin, sres);
  }
}

// Recompute z for one row and one vocabulary tile with the same main loop and
// epilogue arithmetic as bias_tile_kernel.  Called by all 256 threads; wave w
// produces columns 32w..32w+31 of the tile.  ldsArow holds W1[prev] (r elements);
// the row sits at position `row_in_block` (= request or compact row mod 32) of
// its 32-row block, which is where bias_tile_kernel computed it.  Writes z (or
// -inf past V) to zout[0..127].
template <typename T>
__device__ __forceinline__ void recompute_tile_z(const T *ldsArow, const T *W2, const T *Urow,
                                                 int V, int r, int tile, int row_in_block,
                                                 float invT, float *zout) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  floatx16 acc[1][1];
  bias_mainloop<1, 1>(ldsArow, 0, 0, W2, V, r, tile * kTileN + wave * 32, acc);
  const int reg = acc_reg_of_row(row_in_block);
  if ((lane >> 5) == acc_half_of_row(row_in_block)) {
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (e == reg) a = acc[0][0][e];
    const int col = tile * kTileN + wave * 32 + (lane & 31);
    float z = -INFINITY;
    if (col < V) z = (a + Elem<T>::at(Urow, col)) * invT;
    zout[wave * 32 + (lane & 31)] = z;
  }
}

}  // namespace dspark
